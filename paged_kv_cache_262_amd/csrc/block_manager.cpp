// Host-side block manager: the allocator that produces the block tables and
// slot mappings the kernels read.
//
// The KV cache is a pool of fixed-size physical blocks; a sequence's block
// table maps its logical blocks to physical ones, each block carries a
// reference count, and blocks are taken from a free pool on demand as a
// sequence grows and given back when it finishes ("vLLM High-Performance
// Inference Engine: PagedAttention Principles and Deployment Guide", section
// "PagedAttention Architecture Deep Dive" and its block-table example;
// "Configuring vLLM and PagedAttention for High Throughput Enterprise LLM
// Serving", section "Architectural Foundations: PagedAttention & Virtual
// Memory").  Requests with the same prompt prefix share physical blocks, with
// copy-on-write ("vLLM Guide: High-Throughput Multi-GPU LLM Serving with
// PagedAttention", section "What Is PagedAttention?"), and automatic prefix
// caching finds those blocks by hashing the prompt's token blocks (same page,
// section on best practices; "Configuring vLLM ...", section on prefix
// caching).
//
// Policy (deterministic, so tests can replay it):
//   - the free pool is first-in first-out; blocks start in id order;
//   - a sequence takes a new block when its last block is full;
//   - appending to a shared, partly filled last block allocates a new block
//     and records a copy (old -> new) for pa_copy_blocks before the write;
//   - with prefix caching, every full block gets a chained hash of its
//     tokens (the previous block's hash and its own B tokens); a later
//     sequence whose prompt has the same full blocks reuses them.  A hash
//     match alone is never trusted: the block's stored tokens must compare
//     equal and it must follow the same physical block (of the same
//     generation: a block's generation changes whenever the pool hands it
//     out again) as the new sequence's previous block, so by induction the
//     whole prefix, on which the block's keys and values depend, is equal;
//   - a cached block whose count drops to zero stays findable until the free
//     pool hands it out again.
#include <cstdint>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa.h"

namespace {

constexpr uint64_t kFnvOffset = 0xcbf29ce484222325ull;  // FNV-1a, 64-bit
constexpr uint64_t kFnvPrime = 0x100000001b3ull;

uint64_t hash_block(uint64_t prev, const int32_t *tokens, int n) {
    uint64_t h = kFnvOffset;
    auto mix = [&](uint64_t v) {
        for (int i = 0; i < 8; ++i) {
            h ^= (v >> (8 * i)) & 0xff;
            h *= kFnvPrime;
        }
    };
    mix(prev);
    for (int i = 0; i < n; ++i) mix((uint64_t)(uint32_t)tokens[i]);
    return h;
}

struct Block {
    int32_t ref = 0;
    uint32_t gen = 0;             // times the pool has handed this block out
    bool cached = false;          // in the prefix index
    uint64_t hash = 0;
    int32_t parent = -1;          // while cached: the block before it (-1: first block)
    uint32_t parent_gen = 0;
    std::vector<int32_t> tokens;  // the block's tokens while it is cached
};

struct Sequence {
    std::vector<int32_t> table;   // physical block per logical block
    std::vector<int32_t> tokens;  // token ids (for hashing blocks as they fill)
    int64_t len = 0;
    uint64_t last_full_hash = 0;  // chained hash of the last full block (0: none)
};

}  // namespace

struct pa_block_manager {
    int64_t num_blocks = 0;
    int32_t block_size = 0;
    bool prefix_cache = false;
    std::vector<Block> blocks;
    std::deque<int32_t> free_q;          // may hold stale entries (ref > 0): skipped
    std::vector<uint8_t> in_free;        // block id currently counted as free
    int64_t free_count = 0;
    std::unordered_multimap<uint64_t, int32_t> index;  // hash -> cached block
    std::unordered_map<int64_t, Sequence> seqs;
    std::vector<int64_t> copies;         // pending (src, dst) pairs
    int64_t hits = 0;                    // blocks reused from the prefix index

    void uncache(int32_t b) {
        Block &blk = blocks[b];
        if (!blk.cached) return;
        auto range = index.equal_range(blk.hash);
        for (auto it = range.first; it != range.second; ++it)
            if (it->second == b) {
                index.erase(it);
                break;
            }
        blk.cached = false;
        blk.tokens.clear();
    }
    int32_t take_free() {
        while (!free_q.empty()) {
            const int32_t b = free_q.front();
            free_q.pop_front();
            if (!in_free[b]) continue;  // reused from the index meanwhile
            in_free[b] = 0;
            --free_count;
            uncache(b);                 // its old contents are about to be overwritten
            blocks[b].ref = 1;
            ++blocks[b].gen;
            return b;
        }
        return -1;
    }
    void release(int32_t b) {
        if (--blocks[b].ref == 0) {
            in_free[b] = 1;
            ++free_count;
            free_q.push_back(b);
        }
    }
    // The cached block holding exactly these tokens right after block
    // parent (-1: at the start of a sequence), or -1.
    int32_t lookup(uint64_t h, const int32_t *tokens, int32_t parent) const {
        const uint32_t pgen = parent >= 0 ? blocks[parent].gen : 0;
        auto range = index.equal_range(h);
        for (auto it = range.first; it != range.second; ++it) {
            const Block &blk = blocks[it->second];
            if (blk.parent == parent && blk.parent_gen == pgen &&
                std::memcmp(blk.tokens.data(), tokens, sizeof(int32_t) * block_size) == 0)
                return it->second;
        }
        return -1;
    }
    void maybe_cache(Sequence &s, int64_t logical) {
        const int32_t *tok = s.tokens.data() + logical * block_size;
        const uint64_t h = hash_block(s.last_full_hash, tok, block_size);
        s.last_full_hash = h;
        if (!prefix_cache) return;
        const int32_t b = s.table[logical];
        const int32_t parent = logical > 0 ? s.table[logical - 1] : -1;
        if (blocks[b].cached || lookup(h, tok, parent) >= 0) return;  // already indexed
        blocks[b].cached = true;
        blocks[b].hash = h;
        blocks[b].parent = parent;
        blocks[b].parent_gen = parent >= 0 ? blocks[parent].gen : 0;
        blocks[b].tokens.assign(tok, tok + block_size);
        index.emplace(h, b);
    }
};

extern "C" {

pa_status pa_bm_create(int64_t num_blocks, int32_t block_size, int32_t enable_prefix_cache,
                       pa_block_manager **out) {
    if (!out || num_blocks <= 0 || num_blocks > INT32_MAX || block_size <= 0)
        return PA_ERR_INVALID_ARG;
    pa_block_manager *bm = new (std::nothrow) pa_block_manager;
    if (!bm) return PA_ERR_INVALID_ARG;
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->prefix_cache = enable_prefix_cache != 0;
    bm->blocks.resize((size_t)num_blocks);
    bm->in_free.assign((size_t)num_blocks, 1);
    for (int64_t b = 0; b < num_blocks; ++b) bm->free_q.push_back((int32_t)b);
    bm->free_count = num_blocks;
    *out = bm;
    return PA_OK;
}

void pa_bm_destroy(pa_block_manager *bm) { delete bm; }

pa_status pa_bm_add_sequence(pa_block_manager *bm, int64_t seq_id, const int32_t *tokens,
                             int32_t num_tokens, int64_t *slot_mapping,
                             int32_t *num_cached_tokens) {
    if (!bm || num_tokens < 0 || (num_tokens > 0 && (!tokens || !slot_mapping)))
        return PA_ERR_INVALID_ARG;
    if (bm->seqs.count(seq_id)) return PA_ERR_INVALID_ARG;
    const int B = bm->block_size;
    const int64_t nblk = (num_tokens + B - 1) / B;
    // Reuse the leading full blocks the index already holds.
    Sequence s;
    int64_t reused = 0;
    uint64_t h = 0;
    // At most (num_tokens - 1) / B leading blocks are reused, so the prompt's
    // last token always has a slot: its query row must be computed to give
    // the logits of the next token.
    const int64_t max_reuse = num_tokens > 0 ? (num_tokens - 1) / B : 0;
    if (bm->prefix_cache) {
        for (int64_t j = 0; j < max_reuse; ++j) {
            const uint64_t hj = hash_block(h, tokens + j * B, B);
            const int32_t b = bm->lookup(hj, tokens + j * B, j > 0 ? s.table[j - 1] : -1);
            if (b < 0) break;
            h = hj;
            s.table.push_back(b);
            ++reused;
        }
    }
    // Reused blocks that are cached but free (count 0) leave the free pool
    // too: they are counted before any state changes.
    int64_t reclaim = 0;
    for (int64_t j = 0; j < reused; ++j) reclaim += bm->blocks[s.table[j]].ref == 0;
    if (bm->free_count - reclaim < nblk - reused) return PA_ERR_POOL_EXHAUSTED;
    for (int64_t j = 0; j < reused; ++j) {
        const int32_t b = s.table[j];
        if (bm->blocks[b].ref == 0) {  // cached but free: take it back from the pool
            bm->in_free[b] = 0;
            --bm->free_count;
        }
        ++bm->blocks[b].ref;
    }
    bm->hits += reused;
    s.last_full_hash = h;
    for (int64_t j = reused; j < nblk; ++j) s.table.push_back(bm->take_free());
    s.tokens.assign(tokens, tokens + num_tokens);
    s.len = num_tokens;
    for (int32_t t = 0; t < num_tokens; ++t)
        slot_mapping[t] = t < reused * B ? -1
                                         : (int64_t)s.table[t / B] * B + t % B;
    Sequence &ref = bm->seqs.emplace(seq_id, std::move(s)).first->second;
    for (int64_t j = reused; j < num_tokens / B; ++j) bm->maybe_cache(ref, j);
    if (num_cached_tokens) *num_cached_tokens = (int32_t)(reused * B);
    return PA_OK;
}

pa_status pa_bm_append(pa_block_manager *bm, int64_t seq_id, int32_t token, int64_t *slot) {
    if (!bm || !slot) return PA_ERR_INVALID_ARG;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
    Sequence &s = it->second;
    const int B = bm->block_size;
    const int64_t off = s.len % B;
    if (off == 0) {  // a new block
        if (bm->free_count < 1) return PA_ERR_POOL_EXHAUSTED;
        s.table.push_back(bm->take_free());
    } else {
        const int32_t last = s.table.back();
        if (bm->blocks[last].ref > 1) {  // shared and partly filled: copy on write
            if (bm->free_count < 1) return PA_ERR_POOL_EXHAUSTED;
            const int32_t fresh = bm->take_free();
            bm->copies.push_back(last);
            bm->copies.push_back(fresh);
            bm->release(last);
            s.table.back() = fresh;
        }
    }
    *slot = (int64_t)s.table.back() * B + off;
    s.tokens.push_back(token);
    ++s.len;
    if (s.len % B == 0) bm->maybe_cache(s, s.len / B - 1);
    return PA_OK;
}

pa_status pa_bm_fork(pa_block_manager *bm, int64_t parent, int64_t child) {
    if (!bm || parent == child) return PA_ERR_INVALID_ARG;
    auto it = bm->seqs.find(parent);
    if (it == bm->seqs.end() || bm->seqs.count(child)) return PA_ERR_INVALID_ARG;
    Sequence s = it->second;
    for (int32_t b : s.table) ++bm->blocks[b].ref;
    bm->seqs.emplace(child, std::move(s));
    return PA_OK;
}

pa_status pa_bm_free(pa_block_manager *bm, int64_t seq_id) {
    if (!bm) return PA_ERR_INVALID_ARG;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
    for (int32_t b : it->second.table) bm->release(b);
    bm->seqs.erase(it);
    return PA_OK;
}

int32_t pa_bm_take_copies(pa_block_manager *bm, int64_t *pairs, int32_t max_pairs) {
    if (!bm) return -1;
    const int64_t n = (int64_t)bm->copies.size() / 2;
    if (!pairs || max_pairs < n) return (int32_t)n;  // ask again with room for n pairs
    std::memcpy(pairs, bm->copies.data(), sizeof(int64_t) * 2 * n);
    bm->copies.clear();
    return (int32_t)n;
}

pa_status pa_bm_block_table(const pa_block_manager *bm, int64_t seq_id, int32_t *row,
                            int32_t max_blocks, int32_t *num_blocks, int32_t *context_len) {
    if (!bm) return PA_ERR_INVALID_ARG;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
    const Sequence &s = it->second;
    const int32_t n = (int32_t)s.table.size();
    if (num_blocks) *num_blocks = n;
    if (context_len) *context_len = (int32_t)s.len;
    if (row) {
        if (max_blocks < n) return PA_ERR_INVALID_ARG;
        std::memcpy(row, s.table.data(), sizeof(int32_t) * n);
    }
    return PA_OK;
}

pa_status pa_bm_append_batch(pa_block_manager *bm, const int64_t *seq_ids,
                             const int32_t *tokens, int32_t n, int64_t *slots) {
    if (!bm || n < 0 || (n > 0 && (!seq_ids || !tokens || !slots))) return PA_ERR_INVALID_ARG;
    // Blocks the step takes: a new block where the last one is full, a copy
    // where it is shared and partly filled.  Checked up front, so a failed
    // call changes nothing.
    int64_t need = 0;
    std::unordered_set<int64_t> ids;  // one token per sequence: duplicates rejected
    ids.reserve((size_t)n);
    for (int32_t i = 0; i < n; ++i) {
        auto it = bm->seqs.find(seq_ids[i]);
        if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
        if (!ids.insert(seq_ids[i]).second) return PA_ERR_INVALID_ARG;
        const Sequence &sq = it->second;
        if (sq.len % bm->block_size == 0 || bm->blocks[sq.table.back()].ref > 1) ++need;
    }
    if (bm->free_count < need) return PA_ERR_POOL_EXHAUSTED;
    for (int32_t i = 0; i < n; ++i) {
        const pa_status st = pa_bm_append(bm, seq_ids[i], tokens[i], slots + i);
        if (st != PA_OK) return st;  // not reached: checked above
    }
    return PA_OK;
}

pa_status pa_bm_block_tables(const pa_block_manager *bm, const int64_t *seq_ids, int32_t n,
                             int32_t *tables, int32_t max_blocks, int32_t fill,
                             int32_t *context_lens) {
    if (!bm || n < 0 || max_blocks < 0 || (n > 0 && (!seq_ids || !tables))) return PA_ERR_INVALID_ARG;
    for (int32_t i = 0; i < n; ++i) {
        auto it = bm->seqs.find(seq_ids[i]);
        if (it == bm->seqs.end() || (int64_t)it->second.table.size() > max_blocks)
            return PA_ERR_INVALID_ARG;
    }
    for (int32_t i = 0; i < n; ++i) {
        const Sequence &sq = bm->seqs.find(seq_ids[i])->second;
        int32_t *row = tables + (int64_t)i * max_blocks;
        const int32_t nb = (int32_t)sq.table.size();
        std::memcpy(row, sq.table.data(), sizeof(int32_t) * nb);
        for (int32_t j = nb; j < max_blocks; ++j) row[j] = fill;
        if (context_lens) context_lens[i] = (int32_t)sq.len;
    }
    return PA_OK;
}

pa_status pa_bm_get_stats(const pa_block_manager *bm, pa_bm_stats *st) {
    if (!bm || !st) return PA_ERR_INVALID_ARG;
    std::memset(st, 0, sizeof(*st));
    st->num_blocks = bm->num_blocks;
    st->free_blocks = bm->free_count;
    st->used_blocks = bm->num_blocks - bm->free_count;
    for (const Block &b : bm->blocks) {
        if (b.ref > 1) ++st->shared_blocks;
        if (b.cached) ++st->cached_blocks;
    }
    for (const auto &kv : bm->seqs) {
        st->num_seqs += 1;
        st->seq_tokens += kv.second.len;
        st->seq_slots += (int64_t)kv.second.table.size() * bm->block_size;
    }
    st->prefix_hits = bm->hits;
    return PA_OK;
}

}  // extern "C"
