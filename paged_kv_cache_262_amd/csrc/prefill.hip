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
// waves form 4 row groups of 32 rows x 2 key parities: the 64-key blocks of
// the context go in pairs, the even block to 4 waves and the odd one to the
// other 4 (half the LDS traffic per matrix product of 8 waves sharing one
// block).  The two parities' partial softmax states are merged at the end.
//
// Staging.  Key blocks are gathered through the block table straight from
// HBM into LDS (global_load_lds_dwordx4: each lane moves 16 bytes, no
// registers) in two LDS stages that alternate.  K and V rows keep their
// memory layout [key][dim]; the 16-byte chunks of each row are permuted by an
// XOR with a function of the key so that the matrix-operand reads below hit
// distinct LDS banks.  For whole blocks the page address of each 1 KB DMA
// segment is wave-uniform and computed on the scalar unit.
//
// Schedule (bf16).  Each wave runs a two-deep software pipeline over its
// blocks: in step t it computes S^T of its block of pair t, then issues the
// P V products of its block of pair t - 1 one at a time, each with a slice of
// the vector work of the softmax of pair t (row maxima, exponentials, bf16
// packing), so the matrix cores and the vector ALUs work at the same time.
// V is therefore staged one step after K: the stage read in step t holds K of
// pair t and V of pair t - 1, and the DMA issued in step t fills the other
// stage with K of pair t + 1 and V of pair t (the V movers at once, the K
// movers after their S^T products, which keeps the two waves of a SIMD
// balanced).
//
// Products.  They are computed transposed, S^T = K Q^T and O^T = V^T P^T.
// The K operand (16 keys x 32 dims) is one 16-byte LDS read per lane; the
// fp32 S^T tile a lane holds (4 consecutive keys of one row) is, after
// conversion to bf16, exactly the P^T operand the next MFMA needs (the keys
// of the contraction are visited in a fixed permutation shared by both
// operands), so P never goes through LDS; and the V^T operand (16 dims x 8
// keys per lane) comes from row-major V through the transposing LDS read
// ds_read_b64_tr_b16, 4 keys of one dim per read.
#include <type_traits>

#include "pa_common.h"
#include "pa_internal.h"
#include "pa_prefill_append.h"

namespace pa {

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef float floatx4_v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kPfWaves = 8;  // waves per workgroup: 2 key parities x 4 row groups
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
    typedef float floatx2_v __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
    const floatx2_v f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_v));  // RNE
}

// Maxima written as the instructions themselves: fmaxf makes the compiler
// quiet each operand that it cannot prove canonical (every MFMA result)
// with an extra v_max first, which doubles the vector work of the row
// maxima.  A NaN operand is ignored, as by fmaxf; a NaN logit makes its
// weight NaN whatever the maximum is.
__device__ __forceinline__ float vmax2(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Maximum of the 4 NKT logits a lane holds for row tile rt of s[NKT][RT]:
// two values per instruction, in two independent chains.
template <int NKT, int RT>
__device__ __forceinline__ float lane_max(const floatx4_v (&s)[NKT][RT], int rt) {
    constexpr int N = 4 * NKT;
    float a = s[0][rt][0], b = s[0][rt][1];
    int i = 2;
#pragma unroll
    for (; i + 4 <= N; i += 4) {
        a = vmax3(a, s[i / 4][rt][i % 4], s[(i + 1) / 4][rt][(i + 1) % 4]);
        b = vmax3(b, s[(i + 2) / 4][rt][(i + 2) % 4], s[(i + 3) / 4][rt][(i + 3) % 4]);
    }
#pragma unroll
    for (; i + 2 <= N; i += 2) a = vmax3(a, s[i / 4][rt][i % 4], s[(i + 1) / 4][rt][(i + 1) % 4]);
    return vmax2(a, b);
}

// Max of x over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four lanes holding
// one row of an MFMA result), with lane swaps instead of LDS shuffles.
__device__ __forceinline__ float row_max4(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    x = vmax2(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return vmax2(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element i & 3 of the 8-byte pieces addressed by lanes
// (i >> 2) + 4 j, j = 0..3.  Issued as inline assembly so that the compiler
// does not tie it to the DMA in flight into the other stage; its result is
// only read after lds_wait(), which names the registers it completes.
__device__ __forceinline__ s16x4 lds_read_tr16(uint32_t addr) {
    s16x4 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr));
    return r;
}
template <int OFF>
__device__ __forceinline__ s16x4 lds_read_tr16_off(uint32_t addr) {
    s16x4 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}
template <int A, int C>
__device__ __forceinline__ void lds_wait(s16x4 (&v)[A][C][2]) {
    static_assert(A * C == 4, "a batch of eight reads");
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(v[0 / C][0 % C][0]), "+v"(v[0 / C][0 % C][1]), "+v"(v[1 / C][1 % C][0]),
                   "+v"(v[1 / C][1 % C][1]), "+v"(v[2 / C][2 % C][0]), "+v"(v[2 / C][2 % C][1]),
                   "+v"(v[3 / C][3 % C][0]), "+v"(v[3 / C][3 % C][1]));
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// One 64-key block of one tensor in LDS: [key][dim] rows of ROWB bytes.  The
// 16-byte chunk c of row k is stored at chunk position c ^ swz(k).  swz keeps
// bit 0, so the two chunks a transposing read takes stay adjacent, and it
// differs between the rows that share a 256-byte bank window and are read
// together.
template <int D>
struct KvLds {
    static constexpr int ROWB = D * 2;                    // bytes per row
    static constexpr int NCH = ROWB / 16;                 // chunks per row
    static constexpr int KPS = 1024 / ROWB;               // rows per 1 KB DMA segment
    static constexpr int SEGS = kKeyBlock * ROWB / 1024;  // segments per block
    static constexpr int BLOCK_BYTES = kKeyBlock * ROWB;
    static constexpr int STAGE_BYTES = 4 * BLOCK_BYTES;   // K even, K odd, V even, V odd
    static constexpr int SEGS_PER_WAVE = 4 * SEGS / kPfWaves;
    static_assert(4 * SEGS % kPfWaves == 0, "segments split evenly over the waves");
    static __host__ __device__ constexpr int swz(int key) {
        return D == 128 ? (key & 7) << 1 : ((key >> 1) & 3) << 1;
    }
};

// AP (append): new_key / new_value [Tq][Hkv][D] hold the K/V rows of the
// chunks' own tokens (row q_begin + i: position L - n + i of chunk c).  Keys
// at those positions are staged from these rows instead of the pools, and
// every workgroup writes the rows of its own queries (for its kv head) into
// their slots, so the pass needs no cache write before it and no workgroup
// reads a slot another one writes.
template <int D, int B, int G, bool AP>
__global__ __launch_bounds__(kPfWaves * 64) void prefill_chunk_kernel(
    bf16_t *__restrict__ out, const bf16_t *__restrict__ query,
    const bf16_t *__restrict__ key_cache, const bf16_t *__restrict__ value_cache,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ cu_query_lens,
    const int32_t *__restrict__ context_lens, int num_q_heads, int num_kv_heads, int max_blocks,
    int64_t num_blocks, float scale_log2, int num_tiles, int total,
    const bf16_t *__restrict__ new_key, const bf16_t *__restrict__ new_value,
    bf16_t *key_dst, bf16_t *value_dst) {
    using LY = KvLds<D>;
    constexpr int QT = kPfRows / G;  // queries per tile
    constexpr int KS = D / 32;       // k-steps of S^T = K Q^T
    constexpr int DT = D / 16;       // 16-dim tiles of O^T
    constexpr int NRG = kPfWaves / 2;           // row groups
    constexpr int RT = kPfRows / (16 * NRG);    // 16-row tiles per wave
    constexpr int ROWB = LY::ROWB;
    constexpr float NEG_INF = -__builtin_inff();
    static_assert(kPfRows == NRG * RT * 16, "row groups x 2 key parities");

    // Two stages in two distinct LDS arrays: the compiler then knows that the
    // operand reads of one stage do not wait for the DMA filling the other.
    __shared__ __attribute__((aligned(1024))) char stage_a[LY::STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char stage_b[LY::STAGE_BYTES];

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
    const int new0 = L - n;                         // AP: first position of the chunk's rows

    const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
    const int l16 = lane & 15, lg = lane >> 4;
    const int rg = w % NRG, kp = w / NRG;  // row group, key parity

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

    const int64_t block_elems = (int64_t)B * D * num_kv_heads;
    const int64_t block_bytes = block_elems * 2;
    // Table entries at or past this (negative ones included, as unsigned)
    // are outside the pool.
    const uint32_t nb_u32 = (uint32_t)min(num_blocks, (int64_t)1 << 31);
    const int nkb = cdiv(kend, kKeyBlock);
    const int npairs = cdiv(nkb, 2);

    // ---- DMA of one tensor's share of a pair into a stage -------------------
    // A stage holds four 64-key blocks, [K even][K odd][V even][V odd], as
    // 4 * SEGS segments of 1 KB split over the waves: the first half of the
    // waves moves K segments, the other half V segments.  Lane i of a segment
    // moves chunk i % NCH of row i / NCH.  The rows of a segment lie in one
    // page.  For a block wholly inside the tile's keys the page is
    // wave-uniform: its table entry is a scalar load and its address scalar
    // arithmetic, so the vector ALUs, which the softmax needs, do none of this
    // work; the lanes add only their offset inside the segment (which depends
    // only on the segment's parity).  In the tile's last block, keys past kend
    // read the row of key kend - 1 instead (data whose weight is exactly 0),
    // so no LDS row is ever left stale.
    const int seg_row = lane / LY::NCH, seg_ch = lane % LY::NCH;
    static_assert(B % LY::KPS == 0, "a segment's rows share a page");
    static_assert(LY::swz(2 * LY::KPS) == LY::swz(0) && LY::swz(3 * LY::KPS) == LY::swz(LY::KPS),
                  "the chunk permutation of a segment depends on its parity only");
    uint32_t seg_lane_off[2];
#pragma unroll
    for (int par = 0; par < 2; ++par)
        seg_lane_off[par] = (uint32_t)(seg_row * ROWB +
                                       ((seg_ch ^ LY::swz(par * LY::KPS + seg_row)) << 4));
    constexpr int SPW = LY::SEGS_PER_WAVE;
    static_assert(LY::SEGS % SPW == 0, "a wave's segments lie in one block");
    const int dma_tensor = (w * SPW) / (2 * LY::SEGS);  // 0: K, 1: V (uniform)
    auto issue_dma = [&](char *stage, int pr) __attribute__((always_inline)) {
        const int seg0 = w * SPW;
        const int bp = (seg0 / LY::SEGS) & 1, s0 = seg0 % LY::SEGS;
        const int kb = 2 * pr + bp;
        if (kb >= nkb) return;  // block past the tile's keys
        char *dst0 = stage + (dma_tensor * 2 + bp) * LY::BLOCK_BYTES + s0 * 1024;
        const char *pool = (const char *)(dma_tensor ? value_cache : key_cache);
        if (kb * kKeyBlock + kKeyBlock <= (AP ? min(kend, new0) : kend)) {
            const char *head = pool + (int64_t)g * B * D * 2;
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
                const int sg = s0 + j;
                const int key_s = kb * kKeyBlock + sg * LY::KPS;
                uint32_t phys = (uint32_t)bt[key_s / B];
                if (phys >= nb_u32) phys = 0;  // caller error: block 0
                const char *page = head + (int64_t)phys * block_bytes + (key_s % B) * ROWB;
                __builtin_amdgcn_global_load_lds((const void *)(page + seg_lane_off[sg & 1]),
                                                 (lds_void *)(dst0 + j * 1024), 16, 0, 0);
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            const int sg = s0 + j;
            const int kk = sg * LY::KPS + seg_row;
            const int key = min(kb * kKeyBlock + kk, kend - 1);
            const char *src;
            if (AP && key >= new0) {  // one of the chunk's own rows
                const bf16_t *rows = dma_tensor ? new_value : new_key;
                src = (const char *)(rows + ((int64_t)(q_begin + key - new0) * num_kv_heads + g) * D) +
                      ((seg_ch ^ LY::swz(kk)) << 4);
            } else {
                uint32_t phys = (uint32_t)bt[key / B];
                if (phys >= nb_u32) phys = 0;
                src = pool + (int64_t)phys * block_bytes + (((int64_t)g * B + key % B) * D) * 2 +
                      ((seg_ch ^ LY::swz(kk)) << 4);
            }
            __builtin_amdgcn_global_load_lds((const void *)src, (lds_void *)(dst0 + j * 1024), 16,
                                             0, 0);
        }
    };

    // ---- LDS operand addresses (bytes inside a block) -----------------------
    // K operand of key tile kt, k-step ks: row kt * 16 + l16, chunk ks * 4 + lg.
    const int k_row_off = l16 * ROWB;
    const int k_sw = LY::swz(l16);
    // V^T operand of dim tile dt, key half h: the lanes of group lg read rows
    // h * 32 + 4 * lg + (l16 >> 2) (and 16 rows further), dims dt * 16 +
    // 4 * (l16 & 3) .. + 3, i.e. chunk 2 * dt + ((l16 & 3) >> 1), half l16 & 1.
    // The chunk bits of the offset are free in v_row_off, so the swizzled
    // chunk is or-ed in and dim tile dt is an xor of dt << 5.
    const int v_row = 4 * lg + (l16 >> 2);
    const uint32_t v_lane_off = v_row * ROWB + (l16 & 1) * 8 +
                                ((LY::swz(v_row) ^ ((l16 & 3) >> 1)) << 4);

    // ---- the three parts of a block -------------------------------------------
    // S^T = K Q^T for the 64 keys of block Kb: s[kt][rt] holds keys
    // kt * 16 + 4 * lg + i (element i) of row (rg * RT + rt) * 16 + l16.
    constexpr int NKT = kKeyBlock / 16;
    auto qk = [&](const char *Kb, floatx4_v (&s)[NKT][RT]) __attribute__((always_inline)) {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
            u32x4 kf[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kf[ks] = *(const u32x4 *)(Kb + kt * 16 * ROWB + k_row_off +
                                          (((ks * 4 + lg) ^ k_sw) << 4));
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                floatx4_v a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) a = mfma16x16x32(kf[ks], qf[rt][ks], a);
                s[kt][rt] = a;
            }
        }
    };
    // Causal mask: only blocks that reach past the tile's first position need
    // it (a uniform branch).  Masked logits are -inf, never scaled.
    auto mask_s = [&](floatx4_v (&s)[NKT][RT], int key0) __attribute__((always_inline)) {
        if (key0 + kKeyBlock - 1 > pos0) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (key0 + kt * 16 + lg * 4 + i > row_pos[rt]) s[kt][rt][i] = NEG_INF;
        }
    };
    // Reference maximum of row tile rt (log2 units) from its block maximum x.
    // m_row is raised only when a logit exceeds it by more than kPfRescale, so
    // rescales are rare and weights stay below 2^kPfRescale.  alpha brings the
    // accumulators to the new reference; the caller applies it after the
    // products still pending on the old one.  Returns whether alpha may differ
    // from 1 (wave-uniform).
    float mneg[RT];  // -m_row, or 0 while m_row is -inf
    auto new_reference = [&](int rt, float x, float &alpha) __attribute__((always_inline)) -> bool {
        const float cand = x * scale_log2;
        const bool need = __builtin_amdgcn_ballot_w64(cand > m_row[rt] + kPfRescale) != 0;
        const float mn = need ? fmaxf(m_row[rt], cand) : m_row[rt];
        alpha = (!need || m_row[rt] == NEG_INF) ? (need ? 0.f : 1.f) : fast_exp2(m_row[rt] - mn);
        m_row[rt] = mn;
        mneg[rt] = (mn == NEG_INF) ? 0.f : -mn;
        return need;
    };
    // Weight of logit e (row tile e / 16, key tile (e / 4) % 4, element
    // e % 4), kept in s; after every second one the pair is packed into the
    // P^T operand (keys of half kt / 2, word (kt % 2) * 2 + i / 2).
    auto weight = [&](floatx4_v (&s)[NKT][RT], u32x4 (&pn)[RT][2], int e)
                      __attribute__((always_inline)) {
        const int rt = e / 16, kt = (e / 4) % 4, i = e % 4;
        s[kt][rt][i] = fast_exp2(fmaf(s[kt][rt][i], scale_log2, mneg[rt]));
        if (i & 1)
            pn[rt][kt / 2][(kt % 2) * 2 + i / 2] = pack_bf16x2(s[kt][rt][i - 1], s[kt][rt][i]);
    };
    // Transposing reads of V^T for batch b (dim tiles 2b, 2b + 1) of the block
    // at Vb, through the compiler builtin: the address derives from the stage,
    // so no wait for the DMA into the other stage is added.
    typedef s16x4 VBatch[2][2][2];  // [dim tile of the batch][key half][rows +0 / +16]
    auto read_v = [&](const char *Vb, VBatch &dst, int b) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 2; ++r)
                    dst[j][h][r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4 *)(Vb + (v_lane_off ^ ((uint32_t)(2 * b + j) << 5)) +
                                      (2 * h + r) * 16 * ROWB));
    };
    // Product q (0..7) of batch b: O^T of dim tile 2b + q / 4 += V^T P^T over
    // key half (q / 2) % 2, row tile q % 2.
    auto pv_product = [&](const VBatch &v, const u32x4 (&pp)[RT][2], int b, int q)
                          __attribute__((always_inline)) {
        const int j = q / 4, h = (q / 2) % 2, rt = q % 2;
        const s16x8 vf = __builtin_shufflevector(v[j][h][0], v[j][h][1], 0, 1, 2, 3, 4, 5, 6, 7);
        acc_o[2 * b + j][rt] = mfma16x16x32(vf, pp[rt][h], acc_o[2 * b + j][rt]);
    };
    static_assert(RT == 2 && DT % 2 == 0, "two row tiles, dim tiles in pairs");
    constexpr int NB = DT / 2;  // batches of V^T reads
    // The block's second half: O^T += V^T P^T and the row sums (a ones row
    // against the same bf16 P^T the output uses, so numerator and denominator
    // agree) for the weights pp of the previous block, whose V is at Vb (PV),
    // and the softmax of this block's logits s into the weights pn (SM).
    // With both, each matrix product is issued with a slice of the softmax's
    // vector work, and full scheduling barriers keep that order, so the
    // products run on the matrix cores while the maxima and exponentials run
    // on the vector ALUs.  Returns whether the accumulators need the factors
    // alpha (after the products).
    auto pv_softmax = [&](const char *Vb, const u32x4 (&pp)[RT][2], floatx4_v (&s)[NKT][RT],
                          u32x4 (&pn)[RT][2], float (&alpha)[RT], auto pv_tag, auto sm_tag)
                          __attribute__((always_inline)) -> bool {
        constexpr bool PV = decltype(pv_tag)::value, SM = decltype(sm_tag)::value;
        bool any = false;
        if constexpr (!PV) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) any |= new_reference(rt, row_max4(lane_max(s, rt)), alpha[rt]);
#pragma unroll
            for (int e = 0; e < 16 * RT; ++e) weight(s, pn, e);
            return any;
        } else {
            VBatch vb[2];
            read_v(Vb, vb[0], 0);
            if constexpr (!SM) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        acc_l[rt] = mfma16x16x32(ones_row, pp[rt][h], acc_l[rt]);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    if (b + 1 < NB) read_v(Vb, vb[(b + 1) & 1], b + 1);
#pragma unroll
                    for (int q = 0; q < 8; ++q) pv_product(vb[b & 1], pp, b, q);
                }
                return false;
            } else {
                // Row sums and the first batch, with the block maxima.
                float lm[RT], x[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    __builtin_amdgcn_sched_barrier(0);
                    acc_l[rt] = mfma16x16x32(ones_row, pp[rt][0], acc_l[rt]);
                    acc_l[rt] = mfma16x16x32(ones_row, pp[rt][1], acc_l[rt]);
                    lm[rt] = lane_max(s, rt);
                }
                __builtin_amdgcn_sched_barrier(0);
                read_v(Vb, vb[1], 1);
#pragma unroll
                for (int q = 0; q < 8; q += 2) {
                    __builtin_amdgcn_sched_barrier(0);
                    pv_product(vb[0], pp, 0, q);
                    pv_product(vb[0], pp, 0, q + 1);
                    if (q < 2 * RT)
                        x[q / 2] = row_max4(lm[q / 2]);  // products 0-3: lane swaps
                    else  // products 4-7: the new reference maxima
                        any |= new_reference(q / 2 - RT, x[q / 2 - RT], alpha[q / 2 - RT]);
                }
                // The other batches, each product with one or two weights.
#pragma unroll
                for (int b = 1; b < NB; ++b) {
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        __builtin_amdgcn_sched_barrier(0);
                        if (q == 0 && b + 1 < NB) read_v(Vb, vb[(b + 1) & 1], b + 1);
                        pv_product(vb[b & 1], pp, b, q);
                        const int m = (b - 1) * 8 + q, nm = (NB - 1) * 8;
#pragma unroll
                        for (int e = m * 16 * RT / nm; e < (m + 1) * 16 * RT / nm; ++e)
                            weight(s, pn, e);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                return any;
            }
        }
    };

    // ---- main loop -------------------------------------------------------------
    // Step t: S^T of this wave's block of pair t (its K in the current stage),
    // then the P V products of its block of pair t - 1 (that V is in the
    // current stage too) on the matrix cores while the weights of pair t are
    // computed on the vector ALUs.  The DMA issued during step t fills the
    // other stage with K of pair t + 1 and V of pair t, so two stages suffice.
    u32x4 pf[RT][2];  // weights of this wave's block of the previous pair
    auto step = [&](char *cur, char *nxt, int t) __attribute__((always_inline)) {
        __syncthreads();  // cur's DMA landed (every wave waited for its own); nxt is free
        const bool has_s = t < npairs && 2 * t + kp < nkb;
        const bool has_pv = t >= 1 && 2 * (t - 1) + kp < nkb;
        const int dpair = dma_tensor ? t : t + 1;
        const bool dma = dpair < npairs;
        // The V movers (odd parity) issue their share at once, the K movers
        // (even parity) after their S^T products; a wave with no S^T to
        // compute issues it at once.
        const bool late = dma && has_s && kp == 0;
        if (dma && !late) issue_dma(nxt, dpair);
        const char *Kb = cur + kp * LY::BLOCK_BYTES;
        const char *Vb = cur + (2 + kp) * LY::BLOCK_BYTES;
        using yes = std::true_type;
        using no = std::false_type;
        if (has_s) {
            floatx4_v s[NKT][RT];
            qk(Kb, s);
            if (late) issue_dma(nxt, dpair);
            __builtin_amdgcn_sched_barrier(0);
            mask_s(s, (2 * t + kp) * kKeyBlock);
            __builtin_amdgcn_sched_barrier(0);
            float alpha[RT];
            u32x4 pn[RT][2];
            const bool rescale = has_pv ? pv_softmax(Vb, pf, s, pn, alpha, yes{}, yes{})
                                        : pv_softmax(Vb, pf, s, pn, alpha, no{}, yes{});
            if (rescale) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    acc_l[rt] *= alpha[rt];
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) acc_o[dt][rt] *= alpha[rt];
                }
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int h = 0; h < 2; ++h) pf[rt][h] = pn[rt][h];
        } else if (has_pv) {
            floatx4_v s[NKT][RT];
            u32x4 pn[RT][2];
            float alpha[RT];
            pv_softmax(Vb, pf, s, pn, alpha, yes{}, no{});
        }
    };

    if (npairs > 0 && dma_tensor == 0) issue_dma(stage_a, 0);
    for (int t = 0; t <= npairs; t += 2) {
        step(stage_a, stage_b, t);
        if (t + 1 <= npairs) step(stage_b, stage_a, t + 1);
    }
    if (AP) {
        // The K and V rows of this tile's queries (kv head g) into their
        // slots: nq rows of NCH 16-byte chunks per tensor.  Positions before
        // 0 or past the table have no slot; an entry outside the pool is a
        // caller error and is skipped.
        constexpr int NCH = D * 2 / 16;
        for (int t = tid; t < 2 * nq * NCH; t += kPfWaves * 64) {
            const int tensor = t / (nq * NCH), r = (t / NCH) % nq, ch = t % NCH;
            const int pos = pos0 + r;
            if (pos < 0 || pos >= max_tokens) continue;
            const int phys = bt[pos / B];
            if (phys < 0 || (int64_t)phys >= num_blocks) continue;
            const int64_t row = (int64_t)(q_begin + q0 + r) * num_kv_heads + g;
            const u32x4 v = *(const u32x4 *)((tensor ? new_value : new_key) + row * D + ch * 8);
            bf16_t *dstp = (tensor ? value_dst : key_dst) +
                           ((int64_t)phys * block_elems + ((int64_t)g * B + pos % B) * D) + ch * 8;
            *(u32x4 *)dstp = v;
        }
    }
    __syncthreads();  // every wave is done with both stages

    // ---- merge the two key parities, normalise, store ------------------------
    // Each lane of an odd wave hands its (max, sum, O^T fragment) to the lane
    // of the even wave with the same rows; both use the same lane layout.
    static_assert(NRG * 64 * DT * RT * 4 * 4 <= LY::STAGE_BYTES, "merge area");
    // Lane-contiguous: fragment f of a row group's lanes is 64 consecutive
    // 16-byte pieces, so the stores and loads below are free of bank conflicts.
    float *mo = (float *)stage_a + (size_t)rg * 64 * (DT * RT * 4) + lane * 4;
    float *mml = (float *)stage_b + (size_t)rg * 64 * (2 * RT) + lane;
    float lsum[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) lsum[rt] = __shfl(acc_l[rt][0], l16);  // row l16's sum
    if (kp == 1) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) *(floatx4_v *)(mo + (rt * DT + dt) * 256) = acc_o[dt][rt];
            mml[(2 * rt) * 64] = m_row[rt];
            mml[(2 * rt + 1) * 64] = lsum[rt];
        }
    }
    __syncthreads();
    if (kp == 1) return;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const float m1 = mml[(2 * rt) * 64], l1 = mml[(2 * rt + 1) * 64];
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
            const floatx4_v o1 = *(const floatx4_v *)(mo + (rt * DT + dt) * 256);
            const floatx4_v o = (acc_o[dt][rt] * f0 + o1 * f1) * inv;
            uint2 v;
            v.x = pack_bf16x2(o[0], o[1]);
            v.y = pack_bf16x2(o[2], o[3]);
            *(uint2 *)(orow + dt * 16 + lg * 4) = v;
        }
    }
}

// ---------------------------------------------------------------------------
// Prefill chunk over an FP8 (e4m3) cache.
//
// The pools hold e4m3 codes of value / scale, one fp32 scale per pool
// (quantised KV cache: "vLLM Guide: High-Throughput Multi-GPU LLM Serving
// with PagedAttention", the quantisation support among the engine's pillars
// and its FP8 engine example).  K is [block][kv head][token][dim]; V is
// [block][kv head][dim][token], each page transposed.  Every code widens to
// bf16 exactly, so the tiling, products, softmax and merge are those of
// prefill_chunk_kernel; k_scale rides in the softmax scale and v_scale in the
// final normalisation.
//
// Staging (half the bytes of bf16): a 64-key block of K is 64 rows of D bytes,
// moved by DMA with the 16-byte chunks of a row XOR-permuted by the key; a
// block of V is its 64 / B transposed pages, moved as they are (a page is D
// rows of B bytes, one per dim).
//
// Key order.  Row r of 16-key tile kt of a block holds key
// 32 (kt >> 1) + 8 (r >> 2) + (r & 3) + 4 (kt & 1): the S^T fragment a lane
// gets from tiles 2h and 2h + 1 then covers 8 consecutive keys of 32-key half
// h, so its P^T operand pairs with a V^T operand (one dim x 8 keys) that is a
// single 8-byte read of a transposed page row.  The K operand is one D/4-byte
// piece of a key's row per lane (dims lg * D/4 + 8 ks + [0, 8) in k-step ks),
// and Q^T takes the same dims.  Keys past the tile's last key share their V
// words with valid keys; in the tile's last block those bytes are zeroed
// before widening (their weights are 0, their codes may be anything).
// ---------------------------------------------------------------------------

// Two e4m3 codes (bytes 0-1, or 2-3 when HI) -> two bf16, exactly.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// Eight codes (two words, lowest byte first) -> eight bf16.
__device__ __forceinline__ u32x4 e4m3x8_bf16x8(uint32_t w0, uint32_t w1) {
    return u32x4{e4m3x2_bf16x2<false>(w0), e4m3x2_bf16x2<true>(w0), e4m3x2_bf16x2<false>(w1),
                 e4m3x2_bf16x2<true>(w1)};
}

template <int D, int B>
struct KvLds8 {
    static constexpr int NCH = D / 16;                     // 16-byte chunks per K row
    static constexpr int KPS = 1024 / D;                   // K rows per 1 KB DMA segment
    static constexpr int BLOCK_BYTES = kKeyBlock * D;      // 64 keys of K, or of V
    static constexpr int SEGS = BLOCK_BYTES / 1024;        // segments per block
    static constexpr int STAGE_BYTES = 4 * BLOCK_BYTES;    // K even, K odd, V even, V odd
    static constexpr int SEGS_PER_WAVE = 4 * SEGS / kPfWaves;
    static constexpr int PAGE_BYTES = B * D;               // one transposed V page
    static constexpr int SEGS_PER_PAGE = PAGE_BYTES / 1024;
    static_assert(4 * SEGS % kPfWaves == 0, "segments split evenly over the waves");
    static_assert(PAGE_BYTES % 1024 == 0 && B >= KPS, "pages are whole segments");
    // Chunk position of chunk c of K row `key` (inside the block): c ^ swz(key).
    // The 8 lanes of a K read take keys k0 + {0..3, 8..11}; swz maps them to
    // distinct chunks, and with rows of 128 bytes to distinct banks.
    static __host__ __device__ constexpr int swz(int key) {
        return D == 128 ? ((key & 3) | ((key >> 1) & 4)) : ((key >> 3) & 1);
    }
    // The permutation of a K segment's rows depends only on its parity.
    static constexpr bool parity_only() {
        for (int s = 0; s < SEGS; ++s)
            for (int r = 0; r < KPS; ++r)
                if (swz(s * KPS + r) != swz((s & 1) * KPS + r)) return false;
        return true;
    }
};

template <int D, int B, int G>
__global__ __launch_bounds__(kPfWaves * 64) void prefill_chunk_fp8_kernel(
    bf16_t *__restrict__ out, const bf16_t *__restrict__ query,
    const uint8_t *__restrict__ key_cache, const uint8_t *__restrict__ value_cache,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ cu_query_lens,
    const int32_t *__restrict__ context_lens, int num_q_heads, int num_kv_heads, int max_blocks,
    int64_t num_blocks, float scale_log2, float v_scale, int num_tiles, int total) {
    using LY = KvLds8<D, B>;
    constexpr int QT = kPfRows / G;  // queries per tile
    constexpr int KS = D / 32;       // k-steps of S^T = K Q^T
    constexpr int DT = D / 16;       // 16-dim tiles of O^T
    constexpr int KW = D / 64;       // 16-byte K reads per lane and key tile
    constexpr int NRG = kPfWaves / 2;
    constexpr int RT = kPfRows / (16 * NRG);
    constexpr float NEG_INF = -__builtin_inff();
    constexpr int MERGE_BYTES = NRG * 64 * DT * RT * 16;
    constexpr int AREA = LY::STAGE_BYTES > MERGE_BYTES ? LY::STAGE_BYTES : MERGE_BYTES;
    static_assert(kPfRows == NRG * RT * 16, "row groups x 2 key parities");
    static_assert(LY::parity_only(), "segment lane offsets depend on parity only");

    __shared__ __attribute__((aligned(1024))) char stage_a[AREA];
    __shared__ __attribute__((aligned(1024))) char stage_b[AREA];
    __shared__ int bt_s[kBtCache];

    // Workgroup order as in prefill_chunk_kernel: the tiles of one (chunk, kv
    // head) run on one XCD.
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
    const int nq = min(QT, n - q0);
    const int pos0 = L - n + q0;
    const int kend = min(L, pos0 + nq);
    const int32_t *bt = block_tables + (int64_t)c * max_blocks;

    const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
    const int l16 = lane & 15, lg = lane >> 4;
    const int rg = w % NRG, kp = w / NRG;

    // Rows and Q^T operands (dims lg * D/4 + 8 ks + [0, 8) in k-step ks).
    int row_pos[RT];
    bool row_ok[RT];
    u32x4 qf[RT][KS];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = (rg * RT + rt) * 16 + l16;
        const int qi = r / G, hh = r - qi * G;
        row_ok[rt] = qi < nq;
        const int qc = row_ok[rt] ? qi : nq - 1;
        row_pos[rt] = pos0 + qc;
        const bf16_t *qrow = query + ((int64_t)(q_begin + q0 + qc) * num_q_heads + g * G + hh) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[rt][ks] = *(const u32x4 *)(qrow + lg * (D / 4) + ks * 8);
    }

    floatx4_v acc_o[DT][RT];
    floatx4_v acc_l[RT];
    float m_row[RT];
    const u32x4 ones_row = l16 == 0 ? u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u}
                                    : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        m_row[rt] = NEG_INF;
        acc_l[rt] = floatx4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc_o[dt][rt] = floatx4_v{0.f, 0.f, 0.f, 0.f};
    }

    const int64_t page_stride = (int64_t)B * D;  // bytes of one (block, kv head) page
    const int nkb = cdiv(kend, kKeyBlock);
    const int npairs = cdiv(nkb, 2);
    const int nbt = cdiv(kend, B);

    constexpr int kWinBlocks = kBtCache * B / kKeyBlock;
    static_assert(kWinBlocks % 2 == 0, "windows hold whole pairs");
    int win_kb0 = 0, win_p0 = 0;
    auto load_window = [&](int kb0) __attribute__((always_inline)) {
        win_kb0 = kb0;
        win_p0 = kb0 * (kKeyBlock / B);
        const int cnt = min(nbt - win_p0, kBtCache);
        for (int i = tid; i < cnt; i += kPfWaves * 64) bt_s[i] = bt[win_p0 + i];
    };
    auto page_of = [&](int key) __attribute__((always_inline)) -> int64_t {
        int phys = bt_s[key / B - win_p0];
        if (phys < 0 || (int64_t)phys >= num_blocks) phys = 0;  // caller error: block 0
        return ((int64_t)phys * num_kv_heads + g) * page_stride;
    };

    // DMA of one pair of blocks: 4 * SEGS segments of 1 KB ([K even][K odd]
    // [V even][V odd]) split over the waves.  A K segment is KPS rows of one
    // page; lane i moves chunk (i % NCH) ^ swz(row) of row i / NCH into LDS
    // position i.  A V segment is 1 KB of one transposed page, moved as is.
    // Pages past the tile's keys are replaced by the page of key kend - 1 (in
    // V their bytes are zeroed before use), and in the tile's last block each
    // K row past kend reads row kend - 1.
    const int seg_row = lane / LY::NCH, seg_ch = lane % LY::NCH;
    uint32_t seg_lane_off[2];
#pragma unroll
    for (int par = 0; par < 2; ++par)
        seg_lane_off[par] = (uint32_t)(seg_row * D + ((seg_ch ^ LY::swz(par * LY::KPS + seg_row)) << 4));
    const char *kpool = (const char *)key_cache, *vpool = (const char *)value_cache;
    // Offset of the page holding key `key` (a wave-uniform key: the table
    // entry is a scalar load and the offset scalar arithmetic).
    auto page_of_uniform = [&](int key) __attribute__((always_inline)) -> int64_t {
        int phys = bt[key / B];
        if (phys < 0 || (int64_t)phys >= num_blocks) phys = 0;  // caller error: block 0
        return ((int64_t)phys * num_kv_heads + g) * page_stride;
    };
    auto issue_dma = [&](char *stage, int pr) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < LY::SEGS_PER_WAVE; ++j) {
            const int seg = w * LY::SEGS_PER_WAVE + j;  // uniform
            const int tensor = seg / (2 * LY::SEGS), bp = (seg / LY::SEGS) & 1;
            const int s = seg % LY::SEGS;
            const int kb = 2 * pr + bp;
            if (kb >= nkb) continue;
            lds_void *dst = (lds_void *)(stage + (tensor * 2 + bp) * LY::BLOCK_BYTES + s * 1024);
            if (tensor == 1) {
                const int key_p = min(kb * kKeyBlock + (s / LY::SEGS_PER_PAGE) * B, kend - 1);
                const char *base =
                    vpool + page_of_uniform(key_p) + (s % LY::SEGS_PER_PAGE) * 1024;
                __builtin_amdgcn_global_load_lds((const void *)(base + lane * 16), dst, 16, 0, 0);
            } else if (kb * kKeyBlock + kKeyBlock <= kend) {
                const int key_s = kb * kKeyBlock + s * LY::KPS;
                const char *base = kpool + page_of_uniform(key_s) + (key_s % B) * D;
                __builtin_amdgcn_global_load_lds((const void *)(base + seg_lane_off[s & 1]), dst, 16,
                                                 0, 0);
            } else {
                const int kk = s * LY::KPS + seg_row;
                const int key = min(kb * kKeyBlock + kk, kend - 1);
                const char *src = kpool + page_of(key) + (key % B) * D +
                                  ((seg_ch ^ LY::swz(kk)) << 4);
                __builtin_amdgcn_global_load_lds((const void *)src, dst, 16, 0, 0);
            }
        }
    };

    // One 64-key block of this wave's parity.
    auto compute = [&](const char *Kb, const char *Vb, int key0, char *dma_stage, int dma_pair)
                       __attribute__((always_inline)) {
        floatx4_v s[4][RT];
        __builtin_amdgcn_s_setprio(0);  // products at the base priority, softmax raised
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const int key = (kt >> 1) * 32 + 8 * (l16 >> 2) + (l16 & 3) + 4 * (kt & 1);
            u32x4 kraw[KW];
#pragma unroll
            for (int cc = 0; cc < KW; ++cc)
                kraw[cc] = *(const u32x4 *)(Kb + key * D + (((lg * KW + cc) ^ LY::swz(key)) << 4));
            u32x4 kf[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kf[ks] = e4m3x8_bf16x8(kraw[ks >> 1][(ks & 1) * 2], kraw[ks >> 1][(ks & 1) * 2 + 1]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                floatx4_v a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) a = mfma16x16x32(kf[ks], qf[rt][ks], a);
                s[kt][rt] = a;
            }
        }
        __builtin_amdgcn_s_setprio(1);
        // Causal mask (key of element i of tile kt: see the key order above).
        if (key0 + kKeyBlock - 1 > pos0) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (key0 + (kt >> 1) * 32 + 8 * lg + 4 * (kt & 1) + i > row_pos[rt])
                            s[kt][rt][i] = NEG_INF;
        }
        u32x4 pf[RT][2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const float mx = row_max4(lane_max(s, rt));
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
#pragma unroll
            for (int h = 0; h < 2; ++h) acc_l[rt] = mfma16x16x32(ones_row, pf[rt][h], acc_l[rt]);
        }
        if (dma_stage != nullptr) issue_dma(dma_stage, dma_pair);
        __builtin_amdgcn_s_setprio(0);
        // O^T += V^T P^T: dim dt * 16 + l16, keys 32 h + 8 lg + [0, 8).
        const bool tail = key0 + kKeyBlock > kend;
        uint32_t vmask[2][2];  // [half][word]: bytes of keys past kend are cleared
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k0 = key0 + 32 * h + 8 * lg;
            const int cnt = tail ? min(max(kend - k0, 0), 8) : 8;
            vmask[h][0] = cnt >= 4 ? 0xFFFFFFFFu : ((1u << (8 * cnt)) - 1u);
            vmask[h][1] = cnt >= 8 ? 0xFFFFFFFFu : (cnt <= 4 ? 0u : ((1u << (8 * (cnt - 4))) - 1u));
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int d = dt * 16 + l16;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = 32 * h + 8 * lg;  // first key of the lane's 8, inside the block
                const uint2 raw = *(const uint2 *)(Vb + (k / B) * LY::PAGE_BYTES + d * B + (k % B));
                const u32x4 vf = e4m3x8_bf16x8(raw.x & vmask[h][0], raw.y & vmask[h][1]);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    acc_o[dt][rt] = mfma16x16x32(vf, pf[rt][h], acc_o[dt][rt]);
            }
        }
        __builtin_amdgcn_s_setprio(1);
    };

    auto step = [&](char *cur, char *nxt, int pr) __attribute__((always_inline)) {
        __syncthreads();
        const bool next = pr + 1 < npairs;
        if (next && 2 * (pr + 1) + 2 > win_kb0 + kWinBlocks) {
            load_window(2 * (pr + 1));
            __syncthreads();
        }
        const bool works = 2 * pr + kp < nkb;
        const bool late = next && works && kp == 1;
        if (next && !late) issue_dma(nxt, pr + 1);
        if (works)
            compute(cur + kp * LY::BLOCK_BYTES, cur + (2 + kp) * LY::BLOCK_BYTES,
                    (2 * pr + kp) * kKeyBlock, late ? nxt : nullptr, pr + 1);
    };

    load_window(0);
    __syncthreads();
    if (npairs > 0) issue_dma(stage_a, 0);
    for (int pr = 0; pr < npairs; pr += 2) {
        step(stage_a, stage_b, pr);
        if (pr + 1 < npairs) step(stage_b, stage_a, pr + 1);
    }
    __syncthreads();

    // Merge the two key parities, normalise (times v_scale), store.
    // Lane-contiguous: fragment f of a row group's lanes is 64 consecutive
    // 16-byte pieces, so the stores and loads below are free of bank conflicts.
    float *mo = (float *)stage_a + (size_t)rg * 64 * (DT * RT * 4) + lane * 4;
    float *mml = (float *)stage_b + (size_t)rg * 64 * (2 * RT) + lane;
    float lsum[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) lsum[rt] = __shfl(acc_l[rt][0], l16);
    if (kp == 1) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) *(floatx4_v *)(mo + (rt * DT + dt) * 256) = acc_o[dt][rt];
            mml[(2 * rt) * 64] = m_row[rt];
            mml[(2 * rt + 1) * 64] = lsum[rt];
        }
    }
    __syncthreads();
    if (kp == 1) return;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const float m1 = mml[(2 * rt) * 64], l1 = mml[(2 * rt + 1) * 64];
        const float M = fmaxf(m_row[rt], m1);
        const float f0 = (m_row[rt] == NEG_INF) ? 0.f : fast_exp2(m_row[rt] - M);
        const float f1 = (m1 == NEG_INF) ? 0.f : fast_exp2(m1 - M);
        const float l = lsum[rt] * f0 + l1 * f1;
        if (!row_ok[rt]) continue;
        const float inv = l > 0.f ? v_scale / l : 0.f;
        const int r = (rg * RT + rt) * 16 + l16;
        const int qi = r / G, hh = r - qi * G;
        bf16_t *orow = out + ((int64_t)(q_begin + q0 + qi) * num_q_heads + g * G + hh) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const floatx4_v o1 = *(const floatx4_v *)(mo + (rt * DT + dt) * 256);
            const floatx4_v o = (acc_o[dt][rt] * f0 + o1 * f1) * inv;
            uint2 v;
            v.x = pack_bf16x2(o[0], o[1]);
            v.y = pack_bf16x2(o[2], o[3]);
            *(uint2 *)(orow + dt * 16 + lg * 4) = v;
        }
    }
}

template <int D, int B, int G>
static hipError_t launch(const PrefillArgs &a, hipStream_t stream, const void *new_key,
                         const void *new_value) {
    constexpr int QT = kPfRows / G;
    const int tiles = cdiv(a.max_query_len, QT);
    const int64_t total = (int64_t)tiles * a.num_kv_heads * a.num_chunks;
    if (total > 0x7fffffff) return hipErrorInvalidValue;
    if (a.kv_fp8) {
        hipLaunchKernelGGL((prefill_chunk_fp8_kernel<D, B, G>), dim3((unsigned)total),
                           dim3(kPfWaves * 64), 0, stream, (bf16_t *)a.out,
                           (const bf16_t *)a.query, (const uint8_t *)a.key_cache,
                           (const uint8_t *)a.value_cache, a.block_tables, a.cu_query_lens,
                           a.context_lens, a.num_q_heads, a.num_kv_heads, a.max_blocks_per_seq,
                           a.num_blocks, a.scale * kLog2e * a.k_scale, a.v_scale, tiles,
                           (int)total);
        return hipGetLastError();
    }
    if (new_key)
        hipLaunchKernelGGL((prefill_chunk_kernel<D, B, G, true>), dim3((unsigned)total),
                           dim3(kPfWaves * 64), 0, stream, (bf16_t *)a.out,
                           (const bf16_t *)a.query, (const bf16_t *)a.key_cache,
                           (const bf16_t *)a.value_cache, a.block_tables, a.cu_query_lens,
                           a.context_lens, a.num_q_heads, a.num_kv_heads, a.max_blocks_per_seq,
                           a.num_blocks, a.scale * kLog2e, tiles, (int)total,
                           (const bf16_t *)new_key, (const bf16_t *)new_value,
                           (bf16_t *)a.key_cache, (bf16_t *)a.value_cache);
    else
        hipLaunchKernelGGL((prefill_chunk_kernel<D, B, G, false>), dim3((unsigned)total),
                           dim3(kPfWaves * 64), 0, stream, (bf16_t *)a.out,
                           (const bf16_t *)a.query, (const bf16_t *)a.key_cache,
                           (const bf16_t *)a.value_cache, a.block_tables, a.cu_query_lens,
                           a.context_lens, a.num_q_heads, a.num_kv_heads, a.max_blocks_per_seq,
                           a.num_blocks, a.scale * kLog2e, tiles, (int)total,
                           (const bf16_t *)nullptr, (const bf16_t *)nullptr, (bf16_t *)nullptr,
                           (bf16_t *)nullptr);
    return hipGetLastError();
}

template <int D, int B>
static hipError_t by_group(const PrefillArgs &a, hipStream_t stream, const void *nk,
                           const void *nv) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch<D, B, 1>(a, stream, nk, nv);
        case 2: return launch<D, B, 2>(a, stream, nk, nv);
        case 4: return launch<D, B, 4>(a, stream, nk, nv);
        case 8: return launch<D, B, 8>(a, stream, nk, nv);
    }
    return hipErrorNotSupported;
}

template <int D>
static hipError_t by_block(const PrefillArgs &a, hipStream_t stream, const void *nk,
                           const void *nv) {
    switch (a.block_size) {
        case 16: return by_group<D, 16>(a, stream, nk, nv);
        case 32: return by_group<D, 32>(a, stream, nk, nv);
    }
    return hipErrorNotSupported;
}

bool prefill_shape_supported(int head_dim, int block_size, int group) {
    return (head_dim == 64 || head_dim == 128) && (block_size == 16 || block_size == 32) &&
           (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_prefill_chunk(const PrefillArgs &a, hipStream_t stream) {
    switch (a.head_dim) {
        case 64: return by_block<64>(a, stream, nullptr, nullptr);
        case 128: return by_block<128>(a, stream, nullptr, nullptr);
    }
    return hipErrorNotSupported;
}

hipError_t launch_prefill_chunk_append(const PrefillArgs &a, const void *new_key,
                                       const void *new_value, hipStream_t stream) {
    if (a.kv_fp8 || !new_key || !new_value) return hipErrorNotSupported;
    switch (a.head_dim) {
        case 64: return by_block<64>(a, stream, new_key, new_value);
        case 128: return by_block<128>(a, stream, new_key, new_value);
    }
    return hipErrorNotSupported;
}

}  // namespace pa
