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
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pagedattn.h"

struct pa_allocator {
    struct Seq {
        std::vector<int32_t> blocks;
        int32_t len = 0;
    };
    int32_t num_blocks = 0;
    int32_t block_size = 0;
    std::vector<int32_t> free_list;     // taken from the back
    std::vector<int32_t> ref;
    std::unordered_map<int64_t, Seq> seqs;
};

namespace {

int64_t blocks_for(int64_t tokens, int32_t bs) { return (tokens + bs - 1) / bs; }

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
    if (need > (int64_t)a->free_list.size()) return PA_ERR_OUT_OF_BLOCKS;
    pa_allocator::Seq s;
    s.len = num_tokens;
    s.blocks.reserve(need);
    for (int64_t i = 0; i < need; ++i) {
        int32_t b = a->free_list.back();
        a->free_list.pop_back();
        a->ref[b] = 1;
        s.blocks.push_back(b);
    }
    a->seqs.emplace(seq_id, std::move(s));
    return PA_OK;
}

pa_status pa_alloc_fork(pa_allocator* a, int64_t parent_id, int64_t child_id) {
    if (!a) return PA_ERR_INVALID_ARG;
    auto it = a->seqs.find(parent_id);
    if (it == a->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
    if (a->seqs.count(child_id)) return PA_ERR_EXISTS;
    pa_allocator::Seq child = it->second;      // copy of the table, same length
    for (int32_t b : child.blocks) a->ref[b] += 1;
    a->seqs.emplace(child_id, std::move(child));
    return PA_OK;
}

pa_status pa_alloc_append_slots(pa_allocator* a, const int64_t* seq_ids, int32_t n,
                                int64_t* slot_mapping_out, int32_t* cow_pairs_out,
                                int32_t* num_pairs_out) {
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
    if (need > (int64_t)a->free_list.size()) return PA_ERR_OUT_OF_BLOCKS;
    if (copies > 0 && !cow_pairs_out) return PA_ERR_INVALID_ARG;
    int32_t np = 0;
    for (int32_t i = 0; i < n; ++i) {
        pa_allocator::Seq& s = *rows[i];
        const int32_t len = s.len;
        if (len % bs == 0) {                       // earlier blocks full: fresh block
            int32_t b = a->free_list.back();
            a->free_list.pop_back();
            a->ref[b] = 1;
            s.blocks.push_back(b);
        } else {
            int32_t last = s.blocks.back();
            if (a->ref[last] > 1) {                // shared: copy on write
                int32_t b = a->free_list.back();
                a->free_list.pop_back();
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
    }
    *num_pairs_out = np;
    return PA_OK;
}

pa_status pa_alloc_free_seq(pa_allocator* a, int64_t seq_id) {
    if (!a) return PA_ERR_INVALID_ARG;
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
    for (int32_t b : it->second.blocks)
        if (a->ref[b] <= 0) return PA_ERR_REFCOUNT;
    for (int32_t b : it->second.blocks) {
        if (--a->ref[b] == 0) a->free_list.push_back(b);
    }
    a->seqs.erase(it);
    return PA_OK;
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

}  // extern "C"
