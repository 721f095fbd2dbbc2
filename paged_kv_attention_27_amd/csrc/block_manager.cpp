// block_manager.cpp -- host-side KV block manager with full-block prefix
// caching (declared in include/pa.h).
//
// What the pages describe, restated:
//   * a sequence's logical blocks map to physical blocks of a pool reserved up
//     front; allocating or freeing only changes which blocks a request holds
//     ("nano-vLLM offline" course, THE IMPORTANT DETAILS item 02);
//   * the block manager keeps physical block ids, prefix hashes and reference
//     counts ("Nano-vLLM reading notes", key state and module boundaries);
//   * full prefix blocks are shared, the last partial block is not reused, and
//     a block whose count drops to zero keeps its content and can still be hit
//     ("nano-vLLM offline" course, ACCURACY & SCOPE; "Visual atlas" ch.25: a
//     free block is recyclable, not cleared, and may still hit the cache);
//   * cache identity needs more than a token substring ("Visual atlas" ch.28):
//     a block's key chains the key of the block before it and a caller salt.
//
// Design: blocks are recycled least-recently-freed first (a FIFO of free ids),
// so a freed block stays hit-able for as long as possible.  A full block's key
// is a 64-bit hash of (previous key, salt, its tokens); a hit is confirmed by
// comparing the stored tokens, so a hash collision can never share wrong data.
// Once a sequence misses, all its later blocks are fresh (their keys depend on
// every earlier block).  The block holding a prompt's last token is never a
// hit, so a prefill always has at least one query row and only ever writes
// blocks it holds alone.  All state is host memory; nothing touches the GPU.
#include <stdint.h>
#include <string.h>

#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

namespace {

uint64_t mix64(uint64_t x) {   // splitmix64 finaliser
    x += 0x9e3779b97f4a7c15ull;
    x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
    x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
    return x ^ (x >> 31);
}

uint64_t block_key(uint64_t prev, uint64_t salt, const int32_t *tokens, int32_t n) {
    uint64_t h = mix64(prev ^ 0x5bd1e995u) ^ mix64(salt + 0x27d4eb2fu);
    for (int32_t i = 0; i < n; ++i)
        h = mix64(h ^ (uint32_t)tokens[i]);
    return h | 1ull;   // 0 means "no key"
}

struct Block {
    int32_t refs = 0;
    uint64_t key = 0;              // 0: not a registered full block
    uint64_t prev = 0;             // key of the block before it (hit check)
    std::vector<int32_t> tokens;   // content of a registered block (hit check)
};

}  // namespace

struct pa_block_manager {
    int32_t block_size;
    std::vector<Block> blocks;
    std::deque<int32_t> free_ids;                  // refs == 0, oldest-freed first
    std::vector<char> in_free;                     // refs == 0 (entries of free_ids may be stale)
    int32_t free_count = 0;
    std::unordered_map<uint64_t, int32_t> by_key;  // registered full blocks

    // a free block handed out fresh: drop its old registration
    int32_t take_fresh() {
        while (!free_ids.empty()) {
            const int32_t id = free_ids.front();
            free_ids.pop_front();
            if (!in_free[id])
                continue;   // stale entry (the block was revived by a cache hit)
            in_free[id] = 0;
            --free_count;
            Block &b = blocks[id];
            if (b.key) {
                auto it = by_key.find(b.key);
                if (it != by_key.end() && it->second == id)
                    by_key.erase(it);
                b.key = 0;
                b.tokens.clear();
            }
            b.refs = 1;
            return id;
        }
        return -1;
    }

    // a registered full block matching (key, prev, tokens), or -1
    int32_t lookup(uint64_t key, uint64_t prev, const int32_t *tokens) const {
        auto it = by_key.find(key);
        if (it == by_key.end())
            return -1;
        const Block &b = blocks[it->second];
        if (b.prev != prev || (int32_t)b.tokens.size() != block_size ||
            memcmp(b.tokens.data(), tokens, sizeof(int32_t) * block_size) != 0)
            return -1;
        return it->second;
    }

    void reference(int32_t id) {
        Block &b = blocks[id];
        if (b.refs == 0) {
            in_free[id] = 0;   // revived: its free_ids entry becomes stale
            --free_count;
        }
        ++b.refs;
    }

    void register_full(int32_t id, uint64_t key, uint64_t prev, const int32_t *tokens) {
        Block &b = blocks[id];
        b.key = key;
        b.prev = prev;
        b.tokens.assign(tokens, tokens + block_size);
        by_key[key] = id;
    }

    int32_t num_free() const { return free_count; }
};

extern "C" {

pa_block_manager *pa_bm_create(int32_t num_blocks, int32_t block_size)
{
    if (num_blocks < 1 || block_size < 1)
        return nullptr;
    pa_block_manager *bm = new (std::nothrow) pa_block_manager;
    if (!bm)
        return nullptr;
    bm->block_size = block_size;
    bm->blocks.resize(num_blocks);
    bm->in_free.assign(num_blocks, 1);
    bm->free_count = num_blocks;
    for (int32_t i = 0; i < num_blocks; ++i)
        bm->free_ids.push_back(i);
    return bm;
}

void pa_bm_destroy(pa_block_manager *bm) { delete bm; }

int32_t pa_bm_num_free(const pa_block_manager *bm) { return bm ? bm->num_free() : -1; }

int32_t pa_bm_ref_count(const pa_block_manager *bm, int32_t block)
{
    if (!bm || block < 0 || block >= (int32_t)bm->blocks.size())
        return -1;
    return bm->blocks[block].refs;
}

int32_t pa_bm_blocks_needed(const pa_block_manager *bm, const int32_t *tokens, int32_t num_tokens,
                            uint64_t salt)
{
    if (!bm || (num_tokens > 0 && !tokens) || num_tokens < 0)
        return -1;
    const int32_t bs = bm->block_size;
    const int32_t nb = (num_tokens + bs - 1) / bs;
    int32_t need = 0;
    uint64_t prev = 0;
    bool miss = false;
    for (int32_t b = 0; b < nb; ++b) {
        const int32_t n = num_tokens - b * bs < bs ? num_tokens - b * bs : bs;
        if (!miss && n == bs && (b + 1) * bs < num_tokens) {
            const uint64_t key = block_key(prev, salt, tokens + b * bs, bs);
            const int32_t id = bm->lookup(key, prev, tokens + b * bs);
            prev = key;
            if (id >= 0) {
                if (bm->blocks[id].refs == 0)
                    ++need;   // a free cached block still leaves the free pool
                continue;
            }
        }
        miss = true;
        ++need;
    }
    return need;
}

int pa_bm_allocate(pa_block_manager *bm, const int32_t *tokens, int32_t num_tokens, uint64_t salt,
                   int32_t *block_table, int32_t max_blocks, int32_t *num_cached_tokens)
{
    if (!bm || !block_table || !num_cached_tokens || (num_tokens > 0 && !tokens))
        return PA_ERR_NULL;
    const int32_t bs = bm->block_size;
    if (num_tokens < 0)
        return PA_ERR_SHAPE;
    const int32_t nb = (num_tokens + bs - 1) / bs;
    if (nb > max_blocks)
        return PA_ERR_SHAPE;
    const int32_t need = pa_bm_blocks_needed(bm, tokens, num_tokens, salt);
    if (need > bm->num_free())
        return PA_ERR_WORKSPACE;   // not enough free blocks: nothing was taken
    uint64_t prev = 0;
    bool miss = false;
    int32_t cached = 0;
    for (int32_t b = 0; b < nb; ++b) {
        const int32_t *tb = tokens + b * bs;
        const int32_t n = num_tokens - b * bs < bs ? num_tokens - b * bs : bs;
        const uint64_t key = n == bs ? block_key(prev, salt, tb, bs) : 0;
        if (!miss && n == bs && (b + 1) * bs < num_tokens) {
            const int32_t id = bm->lookup(key, prev, tb);
            if (id >= 0) {
                bm->reference(id);
                block_table[b] = id;
                cached += bs;
                prev = key;
                continue;
            }
        }
        miss = true;
        const int32_t id = bm->take_fresh();   // cannot fail: counted above
        block_table[b] = id;
        if (n == bs && bm->lookup(key, prev, tb) < 0)
            bm->register_full(id, key, prev, tb);
        prev = key;
    }
    for (int32_t b = nb; b < max_blocks; ++b)
        block_table[b] = -1;
    *num_cached_tokens = cached;
    return PA_OK;
}

int pa_bm_append(pa_block_manager *bm, const int32_t *tokens, int32_t num_tokens, uint64_t salt,
                 int32_t *block_table, int32_t max_blocks)
{
    if (!bm || !block_table || !tokens)
        return PA_ERR_NULL;
    const int32_t bs = bm->block_size;
    if (num_tokens < 1 || (num_tokens + bs - 1) / bs > max_blocks)
        return PA_ERR_SHAPE;
    const int32_t pos = num_tokens - 1;          // the appended token
    const int32_t lb = pos / bs;
    if (pos % bs == 0) {                         // first token of a new block
        if (block_table[lb] >= 0)
            return PA_ERR_SHAPE;
        const int32_t id = bm->take_fresh();
        if (id < 0)
            return PA_ERR_WORKSPACE;
        block_table[lb] = id;
    } else if (block_table[lb] < 0) {
        return PA_ERR_SHAPE;
    }
    if (pos % bs == bs - 1) {                    // the block just became full: register it
        uint64_t prev = 0;
        for (int32_t b = 0; b < lb; ++b)
            prev = block_key(prev, salt, tokens + b * bs, bs);
        const uint64_t key = block_key(prev, salt, tokens + lb * bs, bs);
        const int32_t id = block_table[lb];
        if (bm->blocks[id].refs == 1 && bm->blocks[id].key == 0 &&
            bm->lookup(key, prev, tokens + lb * bs) < 0)
            bm->register_full(id, key, prev, tokens + lb * bs);
    }
    return PA_OK;
}

int pa_bm_free(pa_block_manager *bm, const int32_t *block_table, int32_t num_blocks)
{
    if (!bm || (num_blocks > 0 && !block_table))
        return PA_ERR_NULL;
    for (int32_t b = num_blocks - 1; b >= 0; --b) {   // last blocks are recycled first
        const int32_t id = block_table[b];
        if (id < 0)
            continue;
        if (id >= (int32_t)bm->blocks.size() || bm->blocks[id].refs <= 0)
            return PA_ERR_SHAPE;
        if (--bm->blocks[id].refs == 0) {
            bm->in_free[id] = 1;
            ++bm->free_count;
            bm->free_ids.push_back(id);
        }
    }
    return PA_OK;
}

}  // extern "C"
