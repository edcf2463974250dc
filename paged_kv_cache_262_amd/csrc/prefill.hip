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
// registers), one pair of blocks ahead of the pair being multiplied, in two
// LDS stages that alternate; the even-parity waves issue their share of it
// before their products, the odd-parity ones after their softmax, so the
// memory pipeline moves it while the matrix cores work.  K and V rows keep their memory layout
// [key][dim]; the 16-byte chunks of each row are permuted by an XOR with a
// function of the key so that the matrix-operand reads below hit distinct
// LDS banks.  The block-table entries of the tile sit in an LDS window.
//
// Products.  They are computed transposed, S^T = K Q^T and O^T = V^T P^T.
// The K operand (16 keys x 32 dims) is one 16-byte LDS read per lane; the
// fp32 S^T tile a lane holds (4 consecutive keys of one row) is, after
// conversion to bf16, exactly the P^T operand the next MFMA needs (the keys
// of the contraction are visited in a fixed permutation shared by both
// operands), so P never goes through LDS; and the V^T operand (16 dims x 8
// keys per lane) comes from row-major V through the transposing LDS read
// ds_read_b64_tr_b16, 4 keys of one dim per read.
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

#ifndef PA_PF_WAVES
#define PA_PF_WAVES 8
#endif
constexpr int kPfWaves = PA_PF_WAVES;  // waves per workgroup: 2 key parities x row groups
constexpr int kPfRows = 128;        // rows (query x head) per workgroup
constexpr int kKeyBlock = 64;       // keys per LDS block
constexpr int kXcds = 8;            // MI355X: 8 accelerator complex dies, one L2 each
constexpr float kPfRescale = 8.0f;  // log2 units
constexpr int kBtCache = 2048;      // block-table entries a tile keeps in LDS
#ifndef PA_PF_HALVES
#define PA_PF_HALVES 2
#endif
constexpr int kPfHalves = PA_PF_HALVES;  // 32-key halves of a block per softmax pass (1 or 2)

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

// Max of x over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four lanes holding
// one row of an MFMA result), with lane swaps instead of LDS shuffles.
__device__ __forceinline__ float row_max4(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
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
    __shared__ int bt_s[kBtCache];

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
    const int nkb = cdiv(kend, kKeyBlock);
    const int npairs = cdiv(nkb, 2);
    const int nbt = cdiv(kend, B);  // pages the tile reads

    // ---- block-table window -------------------------------------------------
    // Entries of pages [win_p0, win_p0 + kBtCache).  It is refilled (rarely:
    // every 32K keys at 16-token pages) before the DMA of a pair it does not
    // cover; barriers separate the refill from the reads on both sides.
    constexpr int kWinBlocks = kBtCache * B / kKeyBlock;
    static_assert(kWinBlocks % 2 == 0, "windows hold whole pairs");
    int win_kb0 = 0, win_p0 = 0;
    auto load_window = [&](int kb0) __attribute__((always_inline)) {
        win_kb0 = kb0;
        win_p0 = kb0 * (kKeyBlock / B);
        const int cnt = min(nbt - win_p0, kBtCache);
        for (int i = tid; i < cnt; i += kPfWaves * 64) bt_s[i] = bt[win_p0 + i];
    };

    // ---- DMA of one pair of key blocks into a stage -------------------------
    // The stage's 4 * SEGS segments of 1 KB ([K even][K odd][V even][V odd])
    // are split over the waves; lane i of a segment moves chunk i % NCH of row
    // i / NCH.  The rows of a segment lie in one page, so each segment is one
    // global_load_lds from a wave-uniform page address plus a per-lane offset
    // that depends only on the segment's parity.  In the tile's last block,
    // keys past kend read the row of key kend - 1 instead (data whose weight
    // is exactly 0), so no LDS row is ever left stale.
    const int seg_row = lane / LY::NCH, seg_ch = lane % LY::NCH;
    static_assert(B % LY::KPS == 0, "a segment's rows share a page");
    static_assert(LY::SEGS_PER_WAVE <= 64, "one lane per segment");
    static_assert(LY::swz(2 * LY::KPS) == LY::swz(0) && LY::swz(3 * LY::KPS) == LY::swz(LY::KPS),
                  "the chunk permutation of a segment depends on its parity only");
    uint32_t seg_lane_off[2];
#pragma unroll
    for (int par = 0; par < 2; ++par)
        seg_lane_off[par] = (uint32_t)(seg_row * ROWB +
                                       ((seg_ch ^ LY::swz(par * LY::KPS + seg_row)) << 4));
    // Lane j < SEGS_PER_WAVE computes the global address of the first row of
    // the wave's segment j of pair pr (its page looked up in the window,
    // out-of-range entries replaced by block 0), all segments in one pass.
    auto lookup_pages = [&](int pr) __attribute__((always_inline)) -> uint64_t {
        const int j = lane < LY::SEGS_PER_WAVE ? lane : 0;
        const int seg = w * LY::SEGS_PER_WAVE + j;
        const int tensor = seg / (2 * LY::SEGS), bp = (seg / LY::SEGS) & 1;
        const int kb = 2 * pr + bp;
        const int key_s = min(kb * kKeyBlock + (seg % LY::SEGS) * LY::KPS, kend - 1);
        int phys = bt_s[key_s / B - win_p0];
        if (phys < 0 || (int64_t)phys >= num_blocks) phys = 0;  // caller error: block 0
        const char *pool = (const char *)(tensor ? value_cache : key_cache);
        return (uint64_t)(uintptr_t)(pool + ((int64_t)phys * block_elems + (int64_t)g * B * D) * 2 +
                                     (key_s % B) * ROWB);
    };
    // This wave's share of the DMA of pair pr into stage (seg_addr from
    // lookup_pages(pr)).
    auto issue_dma = [&](char *stage, int pr, uint64_t seg_addr) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < LY::SEGS_PER_WAVE; ++j) {
            const int seg = w * LY::SEGS_PER_WAVE + j;  // uniform
            const int tensor = seg / (2 * LY::SEGS), bp = (seg / LY::SEGS) & 1;
            const int s = seg % LY::SEGS;
            const int kb = 2 * pr + bp;
            if (kb >= nkb) continue;  // block past the tile's keys
            lds_void *dst = (lds_void *)(stage + (tensor * 2 + bp) * LY::BLOCK_BYTES + s * 1024);
            if (kb * kKeyBlock + kKeyBlock <= (AP ? min(kend, new0) : kend)) {
                const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)seg_addr, j);
                const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(seg_addr >> 32), j);
                const char *page = (const char *)(uintptr_t)(((uint64_t)hi << 32) | lo);
                __builtin_amdgcn_global_load_lds((const void *)(page + seg_lane_off[s & 1]), dst, 16,
                                                 0, 0);
            } else {
                const int kk = s * LY::KPS + seg_row;
                const int key = min(kb * kKeyBlock + kk, kend - 1);
                const char *src;
                if (AP && key >= new0) {  // one of the chunk's own rows
                    const bf16_t *rows = tensor ? new_value : new_key;
                    src = (const char *)(rows + ((int64_t)(q_begin + key - new0) * num_kv_heads +
                                                 g) * D) +
                          ((seg_ch ^ LY::swz(kk)) << 4);
                } else {
                    int phys = bt_s[key / B - win_p0];
                    if (phys < 0 || (int64_t)phys >= num_blocks) phys = 0;
                    const char *pool = (const char *)(tensor ? value_cache : key_cache);
                    src = pool + ((int64_t)phys * block_elems + ((int64_t)g * B + key % B) * D) * 2 +
                          ((seg_ch ^ LY::swz(kk)) << 4);
                }
                __builtin_amdgcn_global_load_lds((const void *)src, dst, 16, 0, 0);
            }
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

    // One 64-key block of this wave's parity: S^T = K Q^T, online softmax,
    // O^T += V^T P^T, in 64 / (32 NH) passes of NH 32-key halves (fewer
    // passes: fewer rescale checks; more: a smaller live S / P^T state).
    // dma_stage != nullptr: issue this wave's share of the DMA of pair
    // dma_pair after the first pass's softmax, before its P V products.
    constexpr int NH = kPfHalves;     // 32-key halves per pass
    constexpr int NKT = 2 * NH;       // 16-key tiles per pass
    constexpr int VB = 4 / NH;        // dim tiles per batch of transposing reads
    static_assert(DT % VB == 0, "dim tiles split into batches");
    auto compute = [&](const char *Kb, const char *Vb, int key0, char *dma_stage, int dma_pair,
                       uint64_t seg_phys) __attribute__((always_inline)) {
        const uint32_t vbase = lds_addr(Vb) + v_lane_off;
#pragma unroll
        for (int hp = 0; hp < 2 / NH; ++hp) {
            const int kt0 = hp * NKT;  // first 16-key tile of the pass
            floatx4_v s[NKT][RT];
            __builtin_amdgcn_s_setprio(0);  // products at the base priority
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                u32x4 kf[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    kf[ks] = *(const u32x4 *)(Kb + (kt0 + kt) * 16 * ROWB + k_row_off +
                                              (((ks * 4 + lg) ^ k_sw) << 4));
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    floatx4_v a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) a = mfma16x16x32(kf[ks], qf[rt][ks], a);
                    s[kt][rt] = a;
                }
            }
            // The softmax runs at a raised priority: the SIMD's other wave
            // keeps the matrix core busy meanwhile, and this wave's vector
            // work is not held back behind it.
            __builtin_amdgcn_s_setprio(1);
            // Causal mask: only passes that reach past the tile's first
            // position need it (a uniform branch).  Masked logits are -inf,
            // never scaled.
            const int pkey0 = key0 + kt0 * 16;
            if (pkey0 + NKT * 16 - 1 > pos0) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (pkey0 + kt * 16 + lg * 4 + i > row_pos[rt]) s[kt][rt][i] = NEG_INF;
            }
            u32x4 pf[RT][NH];  // P^T operands: [rt][32-key half of the pass]
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                float mx = NEG_INF;
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
                    mx = fmaxf(mx, fmaxf(fmaxf(s[kt][rt][0], s[kt][rt][1]),
                                         fmaxf(s[kt][rt][2], s[kt][rt][3])));
                mx = row_max4(mx);
                // The reference maximum m_row (log2 units) is raised only
                // when a logit exceeds it by more than kPfRescale, so the
                // rescale of the accumulators is rare; weights stay below
                // 2^kPfRescale.
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
                float p[NKT][4];
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        p[kt][i] = fast_exp2(fmaf(s[kt][rt][i], scale_log2, mneg));
#pragma unroll
                for (int h = 0; h < NH; ++h) {
                    pf[rt][h][0] = pack_bf16x2(p[2 * h][0], p[2 * h][1]);
                    pf[rt][h][1] = pack_bf16x2(p[2 * h][2], p[2 * h][3]);
                    pf[rt][h][2] = pack_bf16x2(p[2 * h + 1][0], p[2 * h + 1][1]);
                    pf[rt][h][3] = pack_bf16x2(p[2 * h + 1][2], p[2 * h + 1][3]);
                }
                // Row sums on the matrix core: a ones row against the same
                // bf16 P^T the output uses, so numerator and denominator agree.
#pragma unroll
                for (int h = 0; h < NH; ++h)
                    acc_l[rt] = mfma16x16x32(ones_row, pf[rt][h], acc_l[rt]);
            }
            if (hp == 0 && dma_stage != nullptr) issue_dma(dma_stage, dma_pair, seg_phys);
            // O^T += V^T P^T over the pass's halves, VB dim tiles per batch;
            // the transposing reads of the next batch are in flight while the
            // current one multiplies.
            s16x4 vb[2][VB][NH][2];  // [buffer][dim tile of the batch][half][rows +0 / +16]
            auto issue_v = [&](s16x4 (&dst)[VB][NH][2], int dt0) __attribute__((always_inline)) {
#pragma unroll
                for (int j = 0; j < VB; ++j) {
                    const uint32_t a = (vbase + (uint32_t)(hp * NH * 32 * ROWB)) ^
                                       ((uint32_t)(dt0 + j) << 5);
                    dst[j][0][0] = lds_read_tr16(a);
                    dst[j][0][1] = lds_read_tr16_off<16 * ROWB>(a);
                    if constexpr (NH == 2) {
                        dst[j][NH - 1][0] = lds_read_tr16_off<32 * ROWB>(a);
                        dst[j][NH - 1][1] = lds_read_tr16_off<48 * ROWB>(a);
                    }
                }
            };
            issue_v(vb[0], 0);
            __builtin_amdgcn_s_setprio(0);
#pragma unroll
            for (int b = 0; b < DT / VB; ++b) {
                lds_wait(vb[b & 1]);
                if (b + 1 < DT / VB) issue_v(vb[(b + 1) & 1], VB * (b + 1));
#pragma unroll
                for (int j = 0; j < VB; ++j)
#pragma unroll
                    for (int h = 0; h < NH; ++h) {
                        const s16x8 vf = __builtin_shufflevector(vb[b & 1][j][h][0],
                                                                 vb[b & 1][j][h][1], 0, 1, 2, 3,
                                                                 4, 5, 6, 7);
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt)
                            acc_o[VB * b + j][rt] =
                                mfma16x16x32(vf, pf[rt][h], acc_o[VB * b + j][rt]);
                    }
            }
            __builtin_amdgcn_s_setprio(1);
        }
    };

    // One pair: wait for its stage, start the next pair's DMA into the other
    // stage, multiply this wave's block of the pair.  The two waves of a SIMD
    // have different parities: the even one issues its share of the DMA at
    // once, the odd one after its softmax, so the memory pipeline drains one
    // share while the other wave multiplies.
    auto step = [&](char *cur, char *nxt, int pr) __attribute__((always_inline)) {
        __syncthreads();  // cur's DMA landed (every wave waited for its own); nxt is free
        const bool next = pr + 1 < npairs;
        uint64_t seg_phys = 0;
        if (next) {
            if (2 * (pr + 1) + 2 > win_kb0 + kWinBlocks) {
                load_window(2 * (pr + 1));
                __syncthreads();
            }
            seg_phys = lookup_pages(pr + 1);
        }
        const bool works = 2 * pr + kp < nkb;
        const bool late = next && works && kp == 1;
        if (next && !late) issue_dma(nxt, pr + 1, seg_phys);
        if (works)
            compute(cur + kp * LY::BLOCK_BYTES, cur + (2 + kp) * LY::BLOCK_BYTES,
                    (2 * pr + kp) * kKeyBlock, late ? nxt : nullptr, pr + 1, seg_phys);
    };

    load_window(0);
    __syncthreads();
    if (npairs > 0) issue_dma(stage_a, 0, lookup_pages(0));
    for (int pr = 0; pr < npairs; pr += 2) {
        step(stage_a, stage_b, pr);
        if (pr + 1 < npairs) step(stage_b, stage_a, pr + 1);
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
    auto lookup_pages = [&](int pr) __attribute__((always_inline)) -> uint64_t {
        const int j = lane < LY::SEGS_PER_WAVE ? lane : 0;
        const int seg = w * LY::SEGS_PER_WAVE + j;
        const int tensor = seg / (2 * LY::SEGS), bp = (seg / LY::SEGS) & 1, s = seg % LY::SEGS;
        const int kb = 2 * pr + bp;
        if (tensor == 0) {
            const int key_s = min(kb * kKeyBlock + s * LY::KPS, kend - 1);
            return (uint64_t)(uintptr_t)(kpool + page_of(key_s) + (key_s % B) * D);
        }
        const int pg = s / LY::SEGS_PER_PAGE;
        const int key_p = min(kb * kKeyBlock + pg * B, kend - 1);
        return (uint64_t)(uintptr_t)(vpool + page_of(key_p) + (s % LY::SEGS_PER_PAGE) * 1024);
    };
    auto issue_dma = [&](char *stage, int pr, uint64_t seg_addr) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < LY::SEGS_PER_WAVE; ++j) {
            const int seg = w * LY::SEGS_PER_WAVE + j;  // uniform
            const int tensor = seg / (2 * LY::SEGS), bp = (seg / LY::SEGS) & 1;
            const int s = seg % LY::SEGS;
            const int kb = 2 * pr + bp;
            if (kb >= nkb) continue;
            lds_void *dst = (lds_void *)(stage + (tensor * 2 + bp) * LY::BLOCK_BYTES + s * 1024);
            const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)seg_addr, j);
            const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(seg_addr >> 32), j);
            const char *base = (const char *)(uintptr_t)(((uint64_t)hi << 32) | lo);
            if (tensor == 1) {
                __builtin_amdgcn_global_load_lds((const void *)(base + lane * 16), dst, 16, 0, 0);
            } else if (kb * kKeyBlock + kKeyBlock <= kend) {
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
    auto compute = [&](const char *Kb, const char *Vb, int key0, char *dma_stage, int dma_pair,
                       uint64_t seg_phys) __attribute__((always_inline)) {
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
            float mx = NEG_INF;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
                mx = fmaxf(mx, fmaxf(fmaxf(s[kt][rt][0], s[kt][rt][1]),
                                     fmaxf(s[kt][rt][2], s[kt][rt][3])));
            mx = row_max4(mx);
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
        if (dma_stage != nullptr) issue_dma(dma_stage, dma_pair, seg_phys);
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
        uint64_t seg_phys = 0;
        if (next) {
            if (2 * (pr + 1) + 2 > win_kb0 + kWinBlocks) {
                load_window(2 * (pr + 1));
                __syncthreads();
            }
            seg_phys = lookup_pages(pr + 1);
        }
        const bool works = 2 * pr + kp < nkb;
        const bool late = next && works && kp == 1;
        if (next && !late) issue_dma(nxt, pr + 1, seg_phys);
        if (works)
            compute(cur + kp * LY::BLOCK_BYTES, cur + (2 + kp) * LY::BLOCK_BYTES,
                    (2 * pr + kp) * kKeyBlock, late ? nxt : nullptr, pr + 1, seg_phys);
    };

    load_window(0);
    __syncthreads();
    if (npairs > 0) issue_dma(stage_a, 0, lookup_pages(0));
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
