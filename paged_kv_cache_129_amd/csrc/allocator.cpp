// Host block allocator: free list, per-block reference counts, block tables,
// copy-on-write.  Host memory only; no GPU calls.
//
// Rules (each from the pages):
//  * equal-size physical blocks handed out from the END of a free list and
//    given back by appending (KV Cache从原理到实战 §6.2, the paged sketch);
//    a request for more blocks than are free fails before anything is taken;
//  * a sequence takes a new block only when its earlier blocks are full, so
//    it wastes less than one block (KV 缓存与分页注意力 §07 块表);
//  * parallel samples share physical blocks and each block counts its users;
//    before writing into a shared, partly filled block a sequence copies it,
//    writes into the copy and the original's count drops by one; the last
//    holder writes in place (§08 共用，写时复制);
//  * a finished sequence returns its blocks; a block whose count reaches zero
//    goes back to the free list (§07).
//  * prefix caching (§11 后来的做法; KV Cache从原理到实战 §4.2): a full block
//    of a sequence whose token ids are known is identified by its tokens and
//    everything before them — here a 64-bit hash chained over the blocks,
//    checked on every hit against the block's own tokens and its
//    predecessor's hash; a new sequence reuses the longest run of leading
//    full blocks whose identities are held (the first miss ends it); a block
//    whose count drops to zero while its identity is held stays cached in a
//    least-recently-used list (a sequence's later blocks enter it first), and
//    fresh blocks come from the free list first, then from the LRU end of that
//    list, never from blocks in use.
#include <cstdint>
#include <algorithm>
#include <cstring>
#include <list>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pagedattn.h"

struct pa_allocator {
    struct Seq {
        std::vector<int32_t> blocks;
        int32_t len = 0;
        bool tracked = false;            // token ids known (prefix caching applies)
        std::vector<int32_t> tokens;     // when tracked
        std::vector<uint64_t> chain;     // identity hash of each full block, when tracked
    };
    int32_t num_blocks = 0;
    int32_t block_size = 0;
    std::vector<int32_t> free_list;     // taken from the back
    std::vector<int32_t> ref;
    std::unordered_map<int64_t, Seq> seqs;
    // prefix cache: identity hash -> block; per block its identity, predecessor
    // identity and tokens (checked on a hit); cached unreferenced blocks, LRU first
    std::unordered_map<uint64_t, int32_t> cache;
    std::vector<char> registered;
    std::vector<uint64_t> bhash, bparent;
    std::vector<std::vector<int32_t>> btokens;
    std::list<int32_t> lru;
    std::vector<std::list<int32_t>::iterator> lru_pos;
    std::vector<char> in_lru;
    int64_t hit_blocks = 0, evictions = 0;
};

namespace {

int64_t blocks_for(int64_t tokens, int32_t bs) { return (tokens + bs - 1) / bs; }

constexpr uint64_t kChainSeed = 0x243F6A8885A308D3ull;   // identity "before" a first block

uint64_t mix64(uint64_t x) {                            // splitmix64 finaliser
    x += 0x9E3779B97F4A7C15ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

// identity of a full block: its tokens chained onto its predecessor's identity
uint64_t block_identity(uint64_t parent, const int32_t* toks, int32_t bs) {
    uint64_t h = mix64(parent);
    for (int32_t i = 0; i < bs; ++i) h = mix64(h ^ (uint64_t)(uint32_t)toks[i]);
    return h;
}

int64_t available(const pa_allocator* a) { return (int64_t)a->free_list.size() + (int64_t)a->lru.size(); }

void lru_remove(pa_allocator* a, int32_t b) {
    a->lru.erase(a->lru_pos[b]);
    a->in_lru[b] = 0;
}

void unregister(pa_allocator* a, int32_t b) {
    a->cache.erase(a->bhash[b]);
    a->registered[b] = 0;
    a->btokens[b].clear();
}

// a fresh block: the free list first, else the least recently used cached one
int32_t take(pa_allocator* a) {
    if (!a->free_list.empty()) {
        const int32_t b = a->free_list.back();
        a->free_list.pop_back();
        return b;
    }
    const int32_t b = a->lru.front();
    lru_remove(a, b);
    unregister(a, b);
    ++a->evictions;
    return b;
}

// cached block holding full block j of a tracked sequence's tokens, or -1
int32_t lookup(const pa_allocator* a, uint64_t parent, uint64_t h, const int32_t* toks) {
    auto it = a->cache.find(h);
    if (it == a->cache.end()) return -1;
    const int32_t b = it->second;
    if (a->bparent[b] != parent) return -1;
    if (std::memcmp(a->btokens[b].data(), toks, sizeof(int32_t) * a->block_size) != 0) return -1;
    return b;
}

// make full block j of a tracked sequence findable (if its identity is not held
// and the block holds no other identity)
void register_block(pa_allocator* a, const pa_allocator::Seq& s, int32_t j) {
    const int32_t b = s.blocks[j];
    const uint64_t h = s.chain[j];
    if (a->registered[b] || a->cache.count(h)) return;
    a->cache.emplace(h, b);
    a->registered[b] = 1;
    a->bhash[b] = h;
    a->bparent[b] = j == 0 ? kChainSeed : s.chain[j - 1];
    const int32_t* t = s.tokens.data() + (int64_t)j * a->block_size;
    a->btokens[b].assign(t, t + a->block_size);
}

pa_status append_impl(pa_allocator* a, const int64_t* seq_ids, const int32_t* token_ids, int32_t n,
                      int64_t* slot_mapping_out, int32_t* cow_pairs_out, int32_t* num_pairs_out);

}  // namespace

extern "C" {

pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                          pa_allocator** out) {
    if (!out || num_blocks <= 0 || block_size <= 0) return PA_ERR_INVALID_ARG;
    *out = nullptr;
    pa_allocator* a = new (std::nothrow) pa_allocator();
    if (!a) return PA_ERR_INVALID_ARG;
    a->num_blocks = num_blocks;
    a->block_size = block_size;
    a->ref.assign(num_blocks, 0);
    a->registered.assign(num_blocks, 0);
    a->bhash.assign(num_blocks, 0);
    a->bparent.assign(num_blocks, 0);
    a->btokens.resize(num_blocks);
    a->lru_pos.resize(num_blocks);
    a->in_lru.assign(num_blocks, 0);
    a->free_list.resize(num_blocks);
    if (free_order) {
        std::vector<char> seen(num_blocks, 0);
        for (int32_t i = 0; i < num_blocks; ++i) {
            int32_t b = free_order[i];
            if (b < 0 || b >= num_blocks || seen[b]) {
                delete a;
                return PA_ERR_INVALID_ARG;
            }
            seen[b] = 1;
            a->free_list[i] = b;
        }
    } else {
        for (int32_t i = 0; i < num_blocks; ++i) a->free_list[i] = i;
    }
    *out = a;
    return PA_OK;
}

void pa_alloc_destroy(pa_allocator* a) { delete a; }

pa_status pa_alloc_add_seq(pa_allocator* a, int64_t seq_id, int32_t num_tokens) {
    if (!a || num_tokens < 0) return PA_ERR_INVALID_ARG;
    if (a->seqs.count(seq_id)) return PA_ERR_EXISTS;
    int64_t need = blocks_for(num_tokens, a->block_size);
    if (need > available(a)) return PA_ERR_OUT_OF_BLOCKS;
    pa_allocator::Seq s;
    s.len = num_tokens;
    s.blocks.reserve(need);
    for (int64_t i = 0; i < need; ++i) {
        const int32_t b = take(a);
        a->ref[b] = 1;
        s.blocks.push_back(b);
    }
    a->seqs.emplace(seq_id, std::move(s));
    return PA_OK;
}

pa_status pa_alloc_add_seq_tokens(pa_allocator* a, int64_t seq_id, const int32_t* tokens,
                                  int32_t num_tokens, int32_t* num_cached_out) {
    if (!a || num_tokens < 0 || (num_tokens > 0 && !tokens)) return PA_ERR_INVALID_ARG;
    if (a->seqs.count(seq_id)) return PA_ERR_EXISTS;
    const int32_t bs = a->block_size;
    const int32_t full = num_tokens / bs;
    pa_allocator::Seq s;
    s.tracked = true;
    s.tokens.assign(tokens, tokens + num_tokens);
    s.chain.resize(full);
    uint64_t parent = kChainSeed;
    for (int32_t j = 0; j < full; ++j) {
        s.chain[j] = block_identity(parent, tokens + (int64_t)j * bs, bs);
        parent = s.chain[j];
    }
    // longest run of leading full blocks whose identities are cached
    std::vector<int32_t> matched;
    int64_t reclaimed = 0;
    for (int32_t j = 0; j < full; ++j) {
        const int32_t b = lookup(a, j == 0 ? kChainSeed : s.chain[j - 1], s.chain[j],
                                 tokens + (int64_t)j * bs);
        if (b < 0) break;
        matched.push_back(b);
        if (a->ref[b] == 0) ++reclaimed;
    }
    const int64_t need = blocks_for(num_tokens, bs) - (int64_t)matched.size();
    if (need > available(a) - reclaimed) return PA_ERR_OUT_OF_BLOCKS;
    for (int32_t b : matched) {
        if (a->in_lru[b]) lru_remove(a, b);
        a->ref[b] += 1;
    }
    a->hit_blocks += (int64_t)matched.size();
    s.blocks = matched;
    for (int64_t i = 0; i < need; ++i) {
        const int32_t b = take(a);
        a->ref[b] = 1;
        s.blocks.push_back(b);
    }
    s.len = num_tokens;
    for (int32_t j = (int32_t)matched.size(); j < full; ++j) register_block(a, s, j);
    if (num_cached_out) *num_cached_out = (int32_t)matched.size() * bs;
    a->seqs.emplace(seq_id, std::move(s));
    return PA_OK;
}

pa_status pa_alloc_fork(pa_allocator* a, int64_t parent_id, int64_t child_id) {
    if (!a) return PA_ERR_INVALID_ARG;
    auto it = a->seqs.find(parent_id);
    if (it == a->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
    if (a->seqs.count(child_id)) return PA_ERR_EXISTS;
    pa_allocator::Seq child = it->second;      // copy of the table, length and tokens
    for (int32_t b : child.blocks) a->ref[b] += 1;
    a->seqs.emplace(child_id, std::move(child));
    return PA_OK;
}

pa_status pa_alloc_append_slots(pa_allocator* a, const int64_t* seq_ids, int32_t n,
                                int64_t* slot_mapping_out, int32_t* cow_pairs_out,
                                int32_t* num_pairs_out) {
    return append_impl(a, seq_ids, nullptr, n, slot_mapping_out, cow_pairs_out, num_pairs_out);
}

pa_status pa_alloc_append_tokens(pa_allocator* a, const int64_t* seq_ids, const int32_t* token_ids,
                                 int32_t n, int64_t* slot_mapping_out, int32_t* cow_pairs_out,
                                 int32_t* num_pairs_out) {
    if (n > 0 && !token_ids) return PA_ERR_INVALID_ARG;
    return append_impl(a, seq_ids, token_ids, n, slot_mapping_out, cow_pairs_out, num_pairs_out);
}

pa_status pa_alloc_free_seq(pa_allocator* a, int64_t seq_id) {
    if (!a) return PA_ERR_INVALID_ARG;
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
    for (int32_t b : it->second.blocks)
        if (a->ref[b] <= 0) return PA_ERR_REFCOUNT;
    const std::vector<int32_t>& blocks = it->second.blocks;
    for (int32_t b : blocks) --a->ref[b];
    for (int32_t b : blocks)                       // uncached: free list, table order
        if (a->ref[b] == 0 && !a->registered[b]) a->free_list.push_back(b);
    for (auto r = blocks.rbegin(); r != blocks.rend(); ++r) {   // cached: LRU, last block first
        const int32_t b = *r;
        if (a->ref[b] == 0 && a->registered[b] && !a->in_lru[b]) {
            a->lru_pos[b] = a->lru.insert(a->lru.end(), b);
            a->in_lru[b] = 1;
        }
    }
    a->seqs.erase(it);
    return PA_OK;
}

pa_status pa_alloc_swap_out(pa_allocator* dev, pa_allocator* host, int64_t seq_id,
                            int32_t* pairs_out, int32_t max_pairs, int32_t* num_pairs_out) {
    if (!dev || !host || !num_pairs_out || max_pairs < 0 || dev == host) return PA_ERR_INVALID_ARG;
    *num_pairs_out = 0;
    auto it = dev->seqs.find(seq_id);
    if (it == dev->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
    if (host->seqs.count(seq_id)) return PA_ERR_EXISTS;
    if (host->block_size != dev->block_size) return PA_ERR_INVALID_ARG;
    const std::vector<int32_t> table = it->second.blocks;
    if ((int64_t)table.size() > max_pairs || (!table.empty() && !pairs_out)) return PA_ERR_INDEX;
    const pa_status st = pa_alloc_add_seq(host, seq_id, it->second.len);   // all or nothing
    if (st != PA_OK) return st;
    const std::vector<int32_t>& htab = host->seqs.find(seq_id)->second.blocks;
    for (size_t k = 0; k < table.size(); ++k) {
        pairs_out[2 * k] = table[k];
        pairs_out[2 * k + 1] = htab[k];
    }
    *num_pairs_out = (int32_t)table.size();
    return pa_alloc_free_seq(dev, seq_id);
}

pa_status pa_alloc_swap_in(pa_allocator* dev, pa_allocator* host, int64_t seq_id,
                           int32_t* pairs_out, int32_t max_pairs, int32_t* num_pairs_out) {
    if (!dev || !host || !num_pairs_out || max_pairs < 0 || dev == host) return PA_ERR_INVALID_ARG;
    *num_pairs_out = 0;
    auto it = host->seqs.find(seq_id);
    if (it == host->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
    if (dev->seqs.count(seq_id)) return PA_ERR_EXISTS;
    if (host->block_size != dev->block_size) return PA_ERR_INVALID_ARG;
    const std::vector<int32_t> htab = it->second.blocks;
    if ((int64_t)htab.size() > max_pairs || (!htab.empty() && !pairs_out)) return PA_ERR_INDEX;
    const pa_status st = pa_alloc_add_seq(dev, seq_id, it->second.len);     // all or nothing
    if (st != PA_OK) return st;
    const std::vector<int32_t>& dtab = dev->seqs.find(seq_id)->second.blocks;
    for (size_t k = 0; k < htab.size(); ++k) {
        pairs_out[2 * k] = htab[k];
        pairs_out[2 * k + 1] = dtab[k];
    }
    *num_pairs_out = (int32_t)htab.size();
    return pa_alloc_free_seq(host, seq_id);
}

pa_status pa_alloc_export(const pa_allocator* a, const int64_t* seq_ids, int32_t n,
                          int32_t* block_tables_out, int32_t max_blocks,
                          int32_t* context_lens_out) {
    if (!a || n < 0 || max_blocks < 0) return PA_ERR_INVALID_ARG;
    if (n > 0 && (!seq_ids || (!block_tables_out && max_blocks > 0))) return PA_ERR_INVALID_ARG;
    for (int32_t i = 0; i < n; ++i) {
        auto it = a->seqs.find(seq_ids[i]);
        if (it == a->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
        if ((int64_t)it->second.blocks.size() > max_blocks) return PA_ERR_INDEX;
    }
    for (int32_t i = 0; i < n; ++i) {
        const pa_allocator::Seq& s = a->seqs.find(seq_ids[i])->second;
        int32_t* row = block_tables_out + (int64_t)i * max_blocks;
        int32_t k = 0;
        for (; k < (int32_t)s.blocks.size(); ++k) row[k] = s.blocks[k];
        for (; k < max_blocks; ++k) row[k] = -1;
        if (context_lens_out) context_lens_out[i] = s.len;
    }
    return PA_OK;
}

pa_status pa_alloc_physical_block(const pa_allocator* a, int64_t seq_id, int32_t logical_idx,
                                  int32_t* block_out) {
    if (!a || !block_out) return PA_ERR_INVALID_ARG;
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
    if (logical_idx < 0 || logical_idx >= (int32_t)it->second.blocks.size()) return PA_ERR_INDEX;
    *block_out = it->second.blocks[logical_idx];
    return PA_OK;
}

int32_t pa_alloc_num_free(const pa_allocator* a) {
    return a ? (int32_t)a->free_list.size() : -1;
}

int32_t pa_alloc_refcount(const pa_allocator* a, int32_t block) {
    if (!a || block < 0 || block >= a->num_blocks) return -1;
    return a->ref[block];
}

int32_t pa_alloc_seq_len(const pa_allocator* a, int64_t seq_id) {
    if (!a) return -1;
    auto it = a->seqs.find(seq_id);
    return it == a->seqs.end() ? -1 : it->second.len;
}

int32_t pa_alloc_num_seqs(const pa_allocator* a) {
    return a ? (int32_t)a->seqs.size() : -1;
}

int32_t pa_alloc_num_evictable(const pa_allocator* a) {
    return a ? (int32_t)a->lru.size() : -1;
}

pa_status pa_alloc_stats(const pa_allocator* a, pa_alloc_counts* out) {
    if (!a || !out) return PA_ERR_INVALID_ARG;
    const int32_t bs = a->block_size;
    std::vector<int32_t> fill(a->num_blocks, 0);
    for (const auto& kv : a->seqs) {
        const pa_allocator::Seq& s = kv.second;
        for (size_t k = 0; k < s.blocks.size(); ++k) {
            const int64_t f = std::min<int64_t>(bs, std::max<int64_t>(0, (int64_t)s.len - (int64_t)k * bs));
            if (f > fill[s.blocks[k]]) fill[s.blocks[k]] = (int32_t)f;
        }
    }
    int64_t used = 0, filled = 0, cached = 0;
    for (int32_t b = 0; b < a->num_blocks; ++b) {
        if (a->ref[b] > 0) ++used;
        filled += fill[b];
        cached += a->registered[b] ? 1 : 0;
    }
    out->num_blocks = a->num_blocks;
    out->free_blocks = (int64_t)a->free_list.size();
    out->evictable_blocks = (int64_t)a->lru.size();
    out->used_blocks = used;
    out->cached_blocks = cached;
    out->filled_slots = filled;
    out->prefix_hit_blocks = a->hit_blocks;
    out->evictions = a->evictions;
    return PA_OK;
}

}  // extern "C"

namespace {

pa_status append_impl(pa_allocator* a, const int64_t* seq_ids, const int32_t* token_ids, int32_t n,
                      int64_t* slot_mapping_out, int32_t* cow_pairs_out, int32_t* num_pairs_out) {
    if (!a || n < 0 || !num_pairs_out) return PA_ERR_INVALID_ARG;
    if (n > 0 && (!seq_ids || !slot_mapping_out)) return PA_ERR_INVALID_ARG;
    *num_pairs_out = 0;
    const int32_t bs = a->block_size;
    // validate and count the blocks needed before changing anything
    std::vector<pa_allocator::Seq*> rows(n);
    std::unordered_set<int64_t> seen;
    std::unordered_map<int32_t, int32_t> pending;   // copies already planned per shared block
    int64_t need = 0, copies = 0;
    for (int32_t i = 0; i < n; ++i) {
        auto it = a->seqs.find(seq_ids[i]);
        if (it == a->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
        if (!seen.insert(seq_ids[i]).second) return PA_ERR_INVALID_ARG;   // duplicate id
        pa_allocator::Seq& s = it->second;
        if (s.len == INT32_MAX) return PA_ERR_INVALID_ARG;
        rows[i] = &s;
        if (s.len % bs == 0) {
            ++need;
        } else {
            int32_t last = s.blocks.back();
            if (a->ref[last] - pending[last] > 1) {
                ++need;
                ++copies;
                pending[last] += 1;
            }
        }
    }
    if (need > available(a)) return PA_ERR_OUT_OF_BLOCKS;
    if (copies > 0 && !cow_pairs_out) return PA_ERR_INVALID_ARG;
    int32_t np = 0;
    for (int32_t i = 0; i < n; ++i) {
        pa_allocator::Seq& s = *rows[i];
        const int32_t len = s.len;
        if (len % bs == 0) {                       // earlier blocks full: fresh block
            const int32_t b = take(a);
            a->ref[b] = 1;
            s.blocks.push_back(b);
        } else {
            int32_t last = s.blocks.back();
            if (a->ref[last] > 1) {                // shared: copy on write
                const int32_t b = take(a);
                a->ref[last] -= 1;
                a->ref[b] = 1;
                s.blocks.back() = b;
                cow_pairs_out[2 * np] = last;
                cow_pairs_out[2 * np + 1] = b;
                ++np;
            }
        }
        slot_mapping_out[i] = (int64_t)s.blocks[len / bs] * bs + len % bs;
        s.len = len + 1;
        if (!token_ids || !s.tracked) {            // tokens no longer known
            s.tracked = false;
            s.tokens.clear();
            s.chain.clear();
        } else {
            s.tokens.push_back(token_ids[i]);
            if (s.len % bs == 0) {                 // the block is full now: findable
                const int32_t j = len / bs;
                s.chain.push_back(block_identity(j == 0 ? kChainSeed : s.chain[j - 1],
                                                 s.tokens.data() + (int64_t)j * bs, bs));
                register_block(a, s, j);
            }
        }
    }
    *num_pairs_out = np;
    return PA_OK;
}


}  // namespace
