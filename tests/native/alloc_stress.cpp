// Random operation sequences against the host block allocator, built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_allocator_native.py.
// After every call the allocator's state is checked against its invariants:
//   * a block's reference count equals the number of tables that hold it;
//   * free and cached-unreferenced blocks have count 0, and free + cached +
//     held blocks make up the pool;
//   * the counts report agrees (used blocks, evictable blocks);
//   * a sequence of len tokens holds ceil(len / block_size) blocks;
//   * export and physical_block report the same tables;
//   * a failed call changes nothing.
// Exit status 0 when every check holds; the first failure is printed.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "pagedattn.h"

namespace {

int fail(const char* what, uint64_t seed, int step) {
    std::fprintf(stderr, "seed %llu step %d: %s\n", (unsigned long long)seed, step, what);
    return 1;
}

struct Snapshot {
    std::map<int64_t, std::vector<int32_t>> tables;
    std::map<int64_t, int32_t> lens;
    std::vector<int32_t> refs;
    int32_t free_blocks = 0;
    int32_t evictable = 0;
    bool operator==(const Snapshot& o) const {
        return tables == o.tables && lens == o.lens && refs == o.refs &&
               free_blocks == o.free_blocks && evictable == o.evictable;
    }
};

Snapshot snapshot(pa_allocator* a, const std::set<int64_t>& ids, int32_t nb) {
    Snapshot s;
    for (int64_t id : ids) {
        const int32_t len = pa_alloc_seq_len(a, id);
        s.lens[id] = len;
        std::vector<int32_t> row;
        for (int32_t k = 0;; ++k) {
            int32_t b = -1;
            if (pa_alloc_physical_block(a, id, k, &b) != PA_OK) break;
            row.push_back(b);
        }
        s.tables[id] = row;
    }
    for (int32_t b = 0; b < nb; ++b) s.refs.push_back(pa_alloc_refcount(a, b));
    s.free_blocks = pa_alloc_num_free(a);
    s.evictable = pa_alloc_num_evictable(a);
    return s;
}

// the invariants; returns a description of the first one that fails, or null
const char* check(pa_allocator* a, const std::set<int64_t>& ids, int32_t nb, int32_t bs) {
    const Snapshot s = snapshot(a, ids, nb);
    if (pa_alloc_num_seqs(a) != (int32_t)ids.size()) return "sequence count";
    std::vector<int32_t> held(nb, 0);
    for (const auto& kv : s.tables) {
        const int32_t len = s.lens.at(kv.first);
        if (len < 0) return "known sequence reported unknown";
        if ((int64_t)kv.second.size() != ((int64_t)len + bs - 1) / bs) return "table length";
        for (int32_t b : kv.second) {
            if (b < 0 || b >= nb) return "block id out of range";
            held[b] += 1;
        }
    }
    int32_t used = 0;
    for (int32_t b = 0; b < nb; ++b) {
        if (s.refs[b] != held[b]) return "reference count != table occurrences";
        used += held[b] > 0;
    }
    if (used + s.free_blocks + s.evictable != nb) return "free + cached + held != pool";
    pa_alloc_counts c{};
    if (pa_alloc_stats(a, &c) != PA_OK) return "stats failed";
    if (c.used_blocks != used || c.evictable_blocks != s.evictable || c.free_blocks != s.free_blocks ||
        c.num_blocks != nb || c.cached_blocks < c.evictable_blocks)
        return "counts disagree";
    // export agrees with physical_block
    if (!ids.empty()) {
        std::vector<int64_t> v(ids.begin(), ids.end());
        int32_t maxb = 0;
        for (const auto& kv : s.tables) maxb = std::max<int32_t>(maxb, (int32_t)kv.second.size());
        std::vector<int32_t> tab((size_t)v.size() * (maxb + 1), 7), lens(v.size(), 7);
        if (pa_alloc_export(a, v.data(), (int32_t)v.size(), tab.data(), maxb + 1, lens.data()) !=
            PA_OK)
            return "export failed";
        for (size_t i = 0; i < v.size(); ++i) {
            const auto& row = s.tables.at(v[i]);
            if (lens[i] != s.lens.at(v[i])) return "exported length";
            for (int32_t k = 0; k <= maxb; ++k) {
                const int32_t want = k < (int32_t)row.size() ? row[k] : -1;
                if (tab[i * (maxb + 1) + k] != want) return "exported table";
            }
        }
        if (maxb > 0 &&
            pa_alloc_export(a, v.data(), (int32_t)v.size(), tab.data(), maxb - 1, nullptr) !=
                PA_ERR_INDEX)
            return "export into a short table must fail";
    }
    return nullptr;
}

int run(uint64_t seed, int steps) {
    std::mt19937_64 rng(seed);
    auto pick = [&](int n) { return (int)(rng() % (uint64_t)n); };
    const int32_t nb = 1 + pick(48);
    const int32_t bs = 1 << pick(5);
    std::vector<int32_t> order(nb);
    for (int32_t i = 0; i < nb; ++i) order[i] = i;
    std::shuffle(order.begin(), order.end(), rng);
    pa_allocator* a = nullptr;
    if (pa_alloc_create(nb, bs, order.data(), &a) != PA_OK || !a) return fail("create", seed, -1);
    std::set<int64_t> ids;
    int64_t next_id = 0;
    for (int step = 0; step < steps; ++step) {
        const Snapshot before = snapshot(a, ids, nb);
        pa_status st = PA_OK;
        const int op = pick(6);
        std::vector<int64_t> live(ids.begin(), ids.end());
        if (op == 0 || live.empty()) {                         // new sequence
            const int64_t id = pick(8) == 0 && !live.empty() ? live[pick((int)live.size())]
                                                              : next_id++;
            if (pick(2) == 0) {
                st = pa_alloc_add_seq(a, id, pick(3 * bs + 2));
            } else {                                           // with token ids: prefix cache
                std::vector<int32_t> toks(pick(3 * bs + 2) + 1);
                for (auto& t : toks) t = pick(2);
                int32_t cached = -1;
                st = pa_alloc_add_seq_tokens(a, id, toks.data(), (int32_t)toks.size() - 1, &cached);
                if (st == PA_OK && (cached < 0 || cached % bs || cached > (int32_t)toks.size() - 1))
                    return fail("cached token count", seed, step);
            }
            if (st == PA_OK) ids.insert(id);
        } else if (op == 1) {                                  // parallel sample
            const int64_t child = next_id++;
            st = pa_alloc_fork(a, live[pick((int)live.size())], child);
            if (st == PA_OK) ids.insert(child);
        } else if (op == 2 || op == 3) {                       // one decode step
            std::vector<int64_t> batch;
            for (int64_t id : live)
                if (pick(3) != 0) batch.push_back(id);
            if (pick(10) == 0 && !batch.empty()) batch.push_back(batch[0]);   // duplicate id
            if (pick(10) == 0) batch.push_back(next_id + 1000);                // unknown id
            const int32_t n = (int32_t)batch.size();
            std::vector<int64_t> slots(n + 1, -7);
            std::vector<int32_t> pairs(2 * (size_t)n + 2, -7);
            int32_t np = -1;
            const bool no_pairs = pick(8) == 0;
            std::vector<int32_t> toks(n + 1);
            for (auto& t : toks) t = pick(2);
            st = pick(2) == 0 ? pa_alloc_append_slots(a, batch.data(), n, slots.data(),
                                                      no_pairs ? nullptr : pairs.data(), &np)
                              : pa_alloc_append_tokens(a, batch.data(), toks.data(), n, slots.data(),
                                                       no_pairs ? nullptr : pairs.data(), &np);
            if (st == PA_OK) {
                if (np < 0 || np > n) return fail("pair count", seed, step);
                const Snapshot after = snapshot(a, ids, nb);
                std::set<int64_t> seen_slots;
                for (int32_t i = 0; i < n; ++i) {
                    const int32_t len = before.lens.at(batch[i]);
                    if (after.lens.at(batch[i]) != len + 1) return fail("length + 1", seed, step);
                    const int64_t blk = after.tables.at(batch[i])[len / bs];
                    if (slots[i] != blk * bs + len % bs) return fail("slot", seed, step);
                    if (after.refs[blk] != 1) return fail("written block shared", seed, step);
                    if (!seen_slots.insert(slots[i]).second) return fail("slot reused", seed, step);
                }
                std::set<int32_t> dsts;
                for (int32_t p = 0; p < np; ++p) {
                    const int32_t src = pairs[2 * p], dst = pairs[2 * p + 1];
                    if (src == dst || !dsts.insert(dst).second) return fail("pairs", seed, step);
                    if (before.refs[dst] != 0 || before.refs[src] < 2)
                        return fail("copy source not shared or target not free", seed, step);
                }
            }
        } else if (op == 4) {                                  // finished sequence
            const int64_t id = pick(10) == 0 ? next_id + 1000 : live[pick((int)live.size())];
            st = pa_alloc_free_seq(a, id);
            if (st == PA_OK) ids.erase(id);
        } else {                                               // lookups out of range
            int32_t b = 0;
            const int64_t id = live[pick((int)live.size())];
            if (pa_alloc_physical_block(a, id, -1, &b) != PA_ERR_INDEX ||
                pa_alloc_physical_block(a, id, 1 << 20, &b) != PA_ERR_INDEX ||
                pa_alloc_refcount(a, nb) != -1 || pa_alloc_refcount(a, -1) != -1)
                return fail("out-of-range lookups", seed, step);
        }
        if (st != PA_OK && !(snapshot(a, ids, nb) == before))
            return fail("a failed call changed the allocator", seed, step);
        if (const char* why = check(a, ids, nb, bs)) return fail(why, seed, step);
    }
    for (int64_t id : std::vector<int64_t>(ids.begin(), ids.end()))
        if (pa_alloc_free_seq(a, id) != PA_OK) return fail("final free", seed, steps);
    if (pa_alloc_num_free(a) + pa_alloc_num_evictable(a) != nb) return fail("blocks leaked", seed, steps);
    pa_alloc_destroy(a);
    return 0;
}

}  // namespace

int main(int argc, char** argv) {
    const int seeds = argc > 1 ? std::atoi(argv[1]) : 200;
    const int steps = argc > 2 ? std::atoi(argv[2]) : 300;
    // argument errors of create
    pa_allocator* a = nullptr;
    const int32_t dup[3] = {0, 0, 1};
    if (pa_alloc_create(3, 4, dup, &a) != PA_ERR_INVALID_ARG || a)
        return fail("create with a repeated free-order entry", 0, 0);
    if (pa_alloc_create(0, 4, nullptr, &a) != PA_ERR_INVALID_ARG) return fail("create 0", 0, 0);
    if (pa_alloc_num_free(nullptr) != -1 || pa_alloc_num_seqs(nullptr) != -1)
        return fail("null handle", 0, 0);
    for (int s = 0; s < seeds; ++s)
        if (run((uint64_t)s, steps)) return 1;
    std::printf("ok %d seeds x %d steps\n", seeds, steps);
    return 0;
}
