// block_manager.cpp -- host-side block allocator with refcounts, prefix caching and
// copy-on-write, for the paged KV pool the kernels read.
//
// The pool is cut into fixed-size blocks that sequences reference through their block tables
// (page 1, section 4).  Blocks are reference-counted, so sequences that share a prompt prefix
// share its physical blocks (page 2, the PagedAttention section, on sharing across requests).
// Prefix caching works at block granularity: each full block is keyed by a hash chained over
// the block before it and its own token ids, so a later prompt with the same leading tokens
// finds the blocks already computed and only its remainder needs prefill; a partly filled tail
// block is never shared from the cache, which is why common prefixes should end on a block
// boundary (page 1, section 11; page 3, section 2.3).  A sequence that appends into a block
// other sequences still reference first gets a private copy of it (copy-on-write); the caller
// runs the copy on the GPU with pa_copy_blocks before the next append or attention call.
//
// Cached blocks whose refcount drops to zero stay in the cache, evictable, oldest first; an
// allocation takes a never-used or released block first and evicts only when none is left.
// Every hash hit is confirmed by comparing the stored token ids and the parent block, so two
// different prefixes never share a block through a hash collision.
#include <stdint.h>

#include <iterator>
#include <list>
#include <unordered_map>
#include <vector>

#include "pagedattn.h"

namespace {

uint64_t mix64(uint64_t x)
{
    // splitmix64 finaliser (Steele, Lea and Flood, "Fast splittable pseudorandom number generators")
    x += 0x9E3779B97F4A7C15ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

// Hash of a full block: chained over the previous block's hash and this block's token ids.
uint64_t block_hash(uint64_t parent_hash, const int32_t* tokens, int32_t n)
{
    uint64_t h = mix64(parent_hash ^ 0x5851F42D4C957F2Dull);
    for (int32_t i = 0; i < n; i++) h = mix64(h ^ (uint64_t)(uint32_t)tokens[i]);
    return h;
}

constexpr uint64_t kRootHash = 0x243F6A8885A308D3ull;  // parent hash of a sequence's first block

struct Block {
    int32_t ref = 0;
    bool cached = false;       // registered in the prefix map under `hash`
    uint64_t hash = 0;
    int32_t parent = -1;       // block holding the previous tokens of the cached chain
    std::vector<int32_t> tokens;  // token ids of a cached block, to confirm hits
    std::list<int32_t>::iterator lru;  // position in the evictable list when ref == 0 and cached
};

struct Sequence {
    std::vector<int32_t> blocks;    // physical ids, logical order
    std::vector<uint64_t> hashes;   // chain hash of every full block
    std::vector<int32_t> reps;      // the cached block standing for each full block's prefix
    std::vector<int32_t> tail;      // token ids of the partly filled last block
    int32_t num_tokens = 0;
};

}  // namespace

struct pa_block_manager {
    int64_t num_blocks;
    int32_t block_size;
    std::vector<Block> blocks;
    std::vector<int32_t> free_list;  // never used or released uncached blocks (stack)
    std::list<int32_t> evictable;    // cached blocks with refcount 0, oldest release first
    std::unordered_map<uint64_t, int32_t> prefix;  // chain hash -> cached block
    std::unordered_map<int64_t, Sequence> seqs;
    pa_bm_stats stats{};

    int64_t available() const { return (int64_t)free_list.size() + (int64_t)evictable.size(); }

    // Take a block: a free one first, else evict the oldest released cached block.
    int32_t take()
    {
        int32_t b;
        if (!free_list.empty()) {
            b = free_list.back();
            free_list.pop_back();
        } else {
            b = evictable.front();
            evictable.pop_front();
            Block& e = blocks[b];
            auto it = prefix.find(e.hash);
            if (it != prefix.end() && it->second == b) prefix.erase(it);
            e.cached = false;
            e.tokens.clear();
            e.parent = -1;
            stats.evictions++;
        }
        blocks[b].ref = 1;
        return b;
    }

    void release(int32_t b)
    {
        Block& e = blocks[b];
        if (--e.ref > 0) return;
        if (e.cached) {
            evictable.push_back(b);
            e.lru = std::prev(evictable.end());
        } else {
            free_list.push_back(b);
        }
    }

    // A cached block matching (hash, parent, tokens), or -1.
    int32_t lookup(uint64_t h, int32_t parent, const int32_t* tokens) const
    {
        auto it = prefix.find(h);
        if (it == prefix.end()) return -1;
        const Block& e = blocks[it->second];
        if (e.parent != parent || (int32_t)e.tokens.size() != block_size) return -1;
        for (int32_t i = 0; i < block_size; i++)
            if (e.tokens[i] != tokens[i]) return -1;
        return it->second;
    }

    // Register full block b (tokens given, chained after the cached block `parent`) unless its
    // prefix is cached already.  Returns the block that stands for this prefix in the cache: the
    // one found, or b (also when the hash is taken by a different prefix, which stays as it is).
    int32_t register_full(int32_t b, uint64_t h, int32_t parent, const int32_t* tokens)
    {
        if (prefix.count(h)) {
            const int32_t c = lookup(h, parent, tokens);
            return c >= 0 ? c : b;
        }
        Block& e = blocks[b];
        e.cached = true;
        e.hash = h;
        e.parent = parent;
        e.tokens.assign(tokens, tokens + block_size);
        prefix.emplace(h, b);
        return b;
    }
};

extern "C" {

pa_block_manager* pa_bm_create(int64_t num_blocks, int32_t block_size)
{
    if (num_blocks <= 0 || num_blocks > INT32_MAX || block_size <= 0) return nullptr;
    auto* bm = new pa_block_manager();
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->blocks.resize((size_t)num_blocks);
    bm->free_list.reserve((size_t)num_blocks);
    for (int64_t b = num_blocks - 1; b >= 0; b--) bm->free_list.push_back((int32_t)b);  // hands out 0, 1, ...
    return bm;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int32_t pa_bm_add_sequence(pa_block_manager* bm, int64_t seq_id, const int32_t* tokens, int32_t num_tokens,
                           int32_t* cached_tokens)
{
    if (!bm || seq_id < 0 || num_tokens < 0 || (num_tokens > 0 && !tokens) || bm->seqs.count(seq_id))
        return PA_ERR_INVALID_ARG;
    const int32_t B = bm->block_size;
    const int32_t nblk = (num_tokens + B - 1) / B;
    // Leading full blocks found in the cache; at least one prompt token is left to compute.
    const int32_t reusable = num_tokens > 0 ? (num_tokens - 1) / B : 0;
    std::vector<int32_t> hit;
    std::vector<uint64_t> hashes;
    std::vector<int32_t> reps;
    uint64_t h = kRootHash;
    int32_t parent = -1;
    int32_t revived = 0;  // hits that sit in the evictable list
    int64_t lookups = 0;
    for (int32_t i = 0; i < reusable; i++) {
        const uint64_t hi = block_hash(h, tokens + (int64_t)i * B, B);
        lookups++;
        const int32_t b = bm->lookup(hi, parent, tokens + (int64_t)i * B);
        if (b < 0) break;
        hit.push_back(b);
        hashes.push_back(hi);
        reps.push_back(b);
        revived += bm->blocks[b].ref == 0;
        h = hi;
        parent = b;
    }
    const int64_t need = nblk - (int64_t)hit.size();
    if (need > bm->available() - revived) return PA_ERR_NO_BLOCKS;

    Sequence s;
    for (int32_t b : hit) {
        Block& e = bm->blocks[b];
        if (e.ref == 0) bm->evictable.erase(e.lru);
        e.ref++;
        s.blocks.push_back(b);
    }
    bm->stats.lookups += lookups;
    bm->stats.hits += (int64_t)hit.size();
    for (int32_t i = (int32_t)hit.size(); i < nblk; i++) {
        const int32_t b = bm->take();
        s.blocks.push_back(b);
        const int32_t* t = tokens + (int64_t)i * B;
        if ((int64_t)(i + 1) * B <= num_tokens) {  // a full block: register its prefix
            const uint64_t hi = block_hash(h, t, B);
            parent = bm->register_full(b, hi, parent, t);
            hashes.push_back(hi);
            reps.push_back(parent);
            h = hi;
        } else {
            s.tail.assign(t, tokens + num_tokens);
        }
    }
    s.hashes = std::move(hashes);
    s.reps = std::move(reps);
    s.num_tokens = num_tokens;
    bm->seqs.emplace(seq_id, std::move(s));
    if (cached_tokens) *cached_tokens = (int32_t)hit.size() * B;
    return PA_OK;
}

int32_t pa_bm_append_token(pa_block_manager* bm, int64_t seq_id, int32_t token, int64_t* slot, int32_t* copy_src,
                           int32_t* copy_dst)
{
    if (!bm || !slot) return PA_ERR_INVALID_ARG;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
    Sequence& s = it->second;
    const int32_t B = bm->block_size;
    const int32_t o = s.num_tokens % B;
    int32_t src = -1, dst = -1;
    if (o == 0) {  // the token opens a new block
        if (bm->available() < 1) return PA_ERR_NO_BLOCKS;
        s.blocks.push_back(bm->take());
    } else if (bm->blocks[s.blocks.back()].ref > 1) {  // shared partial tail: copy on write
        if (bm->available() < 1) return PA_ERR_NO_BLOCKS;
        src = s.blocks.back();
        dst = bm->take();
        bm->release(src);
        s.blocks.back() = dst;
        bm->stats.cow_copies++;
    }
    *slot = (int64_t)s.blocks.back() * B + o;
    if (copy_src) *copy_src = src;
    if (copy_dst) *copy_dst = dst;
    s.tail.push_back(token);
    s.num_tokens++;
    if ((int32_t)s.tail.size() == B) {  // the block is full: register its prefix
        const uint64_t parent_hash = s.hashes.empty() ? kRootHash : s.hashes.back();
        const int32_t parent = s.reps.empty() ? -1 : s.reps.back();
        const uint64_t hi = block_hash(parent_hash, s.tail.data(), B);
        s.reps.push_back(bm->register_full(s.blocks.back(), hi, parent, s.tail.data()));
        s.hashes.push_back(hi);
        s.tail.clear();
    }
    return PA_OK;
}

int32_t pa_bm_fork(pa_block_manager* bm, int64_t parent_id, int64_t child_id)
{
    if (!bm || child_id < 0 || bm->seqs.count(child_id)) return PA_ERR_INVALID_ARG;
    auto it = bm->seqs.find(parent_id);
    if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
    Sequence c = it->second;
    for (int32_t b : c.blocks) bm->blocks[b].ref++;
    bm->seqs.emplace(child_id, std::move(c));
    return PA_OK;
}

int32_t pa_bm_free_sequence(pa_block_manager* bm, int64_t seq_id)
{
    if (!bm) return PA_ERR_INVALID_ARG;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
    // release from the tail so the chain's head is the last to become evictable
    for (auto b = it->second.blocks.rbegin(); b != it->second.blocks.rend(); ++b) bm->release(*b);
    bm->seqs.erase(it);
    return PA_OK;
}

int32_t pa_bm_block_table(const pa_block_manager* bm, int64_t seq_id, int32_t* table, int32_t max_blocks,
                          int32_t* num_blocks, int32_t* num_tokens)
{
    if (!bm) return PA_ERR_INVALID_ARG;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
    const Sequence& s = it->second;
    if (num_blocks) *num_blocks = (int32_t)s.blocks.size();
    if (num_tokens) *num_tokens = s.num_tokens;
    if (table) {
        if ((int32_t)s.blocks.size() > max_blocks) return PA_ERR_INVALID_ARG;
        for (size_t i = 0; i < s.blocks.size(); i++) table[i] = s.blocks[i];
    }
    return PA_OK;
}

int32_t pa_bm_refcount(const pa_block_manager* bm, int32_t block)
{
    if (!bm || block < 0 || (int64_t)block >= bm->num_blocks) return -1;
    return bm->blocks[block].ref;
}

int32_t pa_bm_get_stats(const pa_block_manager* bm, pa_bm_stats* out)
{
    if (!bm || !out) return PA_ERR_INVALID_ARG;
    *out = bm->stats;
    out->free_blocks = (int64_t)bm->free_list.size();
    out->evictable_blocks = (int64_t)bm->evictable.size();
    out->used_blocks = bm->num_blocks - out->free_blocks - out->evictable_blocks;
    out->cached_blocks = (int64_t)bm->prefix.size();
    return PA_OK;
}

}  // extern "C"
