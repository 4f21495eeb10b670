"""Pins for the oracle allocator's prefix caching, beam-search sharing and
utilisation readout.

The strongest pin is semantic: the allocator is only a bookkeeper, so a
"content model" writes each sequence's token ids into the blocks it was
given fresh (as a prefill or decode step would) and never into blocks it
reused; after every operation, gathering any sequence through its block
table must give back exactly its own token ids.  Reusing a block of another
beginning, evicting a block still in use, or a copy-on-write mistake all
break that.  The pages' own statements (same beginning reused, same block
after another beginning not reused, referenced blocks never evicted, counts
up and down) are checked directly, and planted mistakes must be caught.
"""
import random

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import Allocator, OutOfBlocks
from oracle import allocator as oalloc


def kv_of(tokens, t):
    """Stand-in for the key/value of token t: it depends on the token and on
    everything before it (position and context), as real keys and values do."""
    return hash(tuple(tokens[:t + 1]))


class ContentModel:
    """Pool contents (stand-in keys/values), written only where the caller would write."""

    def __init__(self, alloc):
        self.a = alloc
        self.pool = np.full((alloc.num_blocks, alloc.block_size), -1, dtype=np.int64)
        self.tokens = {}

    def add(self, sid, tokens):
        cached = self.a.add_seq_tokens(sid, tokens)
        table = self.a.tables[sid]
        bs = self.a.block_size
        for t in range(cached, len(tokens)):          # prefill writes the uncached tokens only
            self.pool[table[t // bs], t % bs] = kv_of(tokens, t)
        self.tokens[sid] = list(tokens)
        return cached

    def fork(self, parent, child):
        self.a.fork(parent, child)
        self.tokens[child] = list(self.tokens[parent])

    def append(self, sids, toks):
        slots, pairs = self.a.append_slots(sids, toks)
        for src, dst in pairs:                         # copy-on-write copies first
            self.pool[dst] = self.pool[src]
        bs = self.a.block_size
        for sid, slot, tok in zip(sids, slots, toks):
            self.tokens[sid].append(tok)
            self.pool[slot // bs, slot % bs] = kv_of(self.tokens[sid], len(self.tokens[sid]) - 1)

    def free(self, sid):
        self.a.free_seq(sid)
        del self.tokens[sid]

    def check(self):
        bs = self.a.block_size
        for sid, toks in self.tokens.items():
            table = self.a.tables[sid]
            got = [int(self.pool[table[t // bs], t % bs]) for t in range(len(toks))]
            assert got == [kv_of(toks, t) for t in range(len(toks))], sid
        a = self.a
        used = {b for b in range(a.num_blocks) if a.ref[b] > 0}
        assert set(a.free).isdisjoint(used) and set(a.evictable).isdisjoint(used)
        assert set(a.free).isdisjoint(a.evictable)
        assert len(a.free) + len(a.evictable) + len(used) == a.num_blocks
        assert set(a.evictable) == {b for b in a.block_key if a.ref[b] == 0}
        occurrences = np.zeros(a.num_blocks, dtype=np.int64)
        for table in a.tables.values():
            for b in table:
                occurrences[b] += 1
        assert occurrences.tolist() == a.ref


def test_same_beginning_reuses_blocks():
    """Requests that begin alike reuse the cached full blocks of that beginning
    (KV 缓存与分页注意力 §11): 3 shared full blocks of 4 tokens, then each its own."""
    a = Allocator(32, 4)
    cm = ContentModel(a)
    prompt = list(range(100, 112))                      # 3 full blocks
    assert cm.add(1, prompt + [7, 8]) == 0
    assert cm.add(2, prompt + [9]) == 12
    assert a.tables[2][:3] == a.tables[1][:3] and a.tables[2][3] != a.tables[1][3]
    assert [a.refcount(b) for b in a.tables[1][:3]] == [2, 2, 2]
    assert a.stats()["prefix_hit_blocks"] == 3
    cm.check()


def test_same_block_after_another_beginning_is_not_reused():
    """The same words at another position have other keys and values (§12): a block
    with equal tokens but a different beginning is a different block."""
    a = Allocator(32, 4)
    cm = ContentModel(a)
    cm.add(1, [1, 2, 3, 4, 5, 6, 7, 8])
    assert cm.add(2, [9, 9, 9, 9, 5, 6, 7, 8]) == 0     # second block equal, first not
    assert cm.add(3, [1, 2, 3, 4, 0, 0, 0, 0]) == 4     # only the first block
    assert cm.add(4, [1, 2, 3, 4, 5, 6, 7, 8, 1]) == 8  # both, then its own partial block
    cm.check()


def test_referenced_blocks_never_evicted_and_lru_order():
    """Cached blocks outlive their sequences until space is needed; eviction takes
    the least recently released unreferenced block, never one in use (KV Cache从原理
    到实战 §4.2)."""
    a = Allocator(6, 2)
    cm = ContentModel(a)
    cm.add(1, [1, 1, 2, 2])              # blocks A, B
    cm.add(2, [3, 3])                    # block C
    cm.free(1)                           # A, B cached, unreferenced (B first in LRU)
    assert a.num_free() == 3 and a.num_evictable() == 2
    cm.free(2)                           # C cached after them
    lru = list(a.evictable)
    assert lru == [a.cache[(1, 1, 2, 2)], a.cache[(1, 1)], a.cache[(3, 3)]]
    cm.add(3, [9, 9, 9, 9, 9, 9, 9, 9])  # 4 blocks: 3 free + the least recent cached
    assert a.stats()["evictions"] == 1 and (1, 1, 2, 2) not in a.cache     # B went
    assert a.block_key[lru[1]] == (1, 1) and a.block_key[lru[2]] == (3, 3)  # A, C kept
    assert cm.add(4, [1, 1, 2, 2]) == 2                                      # A reused
    cm.check()
    # with every block referenced, a request that needs more fails and changes nothing
    before = (list(a.free), list(a.evictable), list(a.ref))
    with pytest.raises(OutOfBlocks):
        cm.add(5, list(range(20)))
    assert (list(a.free), list(a.evictable), list(a.ref)) == before
    cm.check()


def test_reuse_of_an_evictable_block_takes_it_back():
    a = Allocator(8, 4)
    cm = ContentModel(a)
    cm.add(1, list(range(8)))
    cm.free(1)
    assert a.num_evictable() == 2
    assert cm.add(2, list(range(8)) + [50]) == 8
    assert a.num_evictable() == 0 and a.refcount(a.tables[2][0]) == 1
    cm.check()


def test_blocks_filled_by_decoding_become_findable():
    a = Allocator(16, 4)
    cm = ContentModel(a)
    cm.add(1, [5, 6])
    cm.append([1], [7])
    cm.append([1], [8])                                  # block 0 full now: registered
    assert cm.add(2, [5, 6, 7, 8, 1]) == 4
    cm.check()


def test_beam_search_shares_and_copies_on_write():
    """Beam search: beams fork from a common history, the pruned ones are freed,
    writes into a shared partly filled block copy it first (§08).  Shared blocks
    make the beams hold fewer blocks than separate copies would."""
    rng = random.Random(3)
    a = Allocator(200, 4)
    cm = ContentModel(a)
    cm.add(0, [1, 2, 3, 4, 5, 6])
    beams, nxt = [0], 1
    peak_shared, peak_separate = 0, 0
    for step in range(12):
        cand = []
        for b in beams:                                  # each beam proposes 3 children
            for _ in range(3):
                cm.fork(b, nxt)
                cand.append(nxt)
                nxt += 1
        for b in beams:
            cm.free(b)
        keep = rng.sample(cand, min(4, len(cand)))       # width 4
        for c in cand:
            if c not in keep:
                cm.free(c)
        beams = keep
        cm.append(beams, [rng.randrange(50) for _ in beams])
        cm.check()
        used = sum(1 for r in a.ref if r > 0)
        separate = sum(len(a.tables[b]) for b in beams)
        peak_shared, peak_separate = max(peak_shared, used), max(peak_separate, separate)
    assert peak_shared < peak_separate


@settings(max_examples=200, deadline=None)
@given(seed=st.integers(0, 10_000), nb=st.integers(4, 40), bs=st.sampled_from([1, 2, 4]))
def test_random_operations_keep_contents_and_invariants(seed, nb, bs):
    rng = random.Random(seed)
    a = Allocator(nb, bs, list(np.random.default_rng(seed).permutation(nb)))
    cm = ContentModel(a)
    prompts = [[rng.randrange(3) for _ in range(rng.randrange(0, 10))] for _ in range(5)]
    nxt = 0
    for _ in range(40):
        op = rng.randrange(5)
        live = list(cm.tokens)
        try:
            if op == 0 or not live:
                p = list(rng.choice(prompts)) + [rng.randrange(3) for _ in range(rng.randrange(3))]
                cm.add(nxt, p)
                nxt += 1
            elif op == 1:
                cm.fork(rng.choice(live), nxt)
                nxt += 1
            elif op == 2:
                sids = rng.sample(live, rng.randrange(1, len(live) + 1))
                cm.append(sids, [rng.randrange(3) for _ in sids])
            else:
                cm.free(rng.choice(live))
        except OutOfBlocks:
            pass
        cm.check()


def test_planted_mistakes_are_caught(monkeypatch):
    """An identity that forgets the beginning, or eviction that takes a block
    still in use, must break the content check."""
    def run():
        a = Allocator(5, 2)
        cm = ContentModel(a)
        cm.add(1, [1, 2, 3, 4])
        cm.add(2, [3, 4, 9, 9])          # (3, 4) again, but at the start
        cm.add(3, [1, 2])
        cm.check()

    run()                                               # the model as written passes
    monkeypatch.setattr(oalloc.Allocator, "_identity",
                        lambda self, tokens, j: tuple(tokens[j * self.block_size:(j + 1) * self.block_size]))
    with pytest.raises(AssertionError):
        run()
    monkeypatch.undo()

    def greedy_take(self):
        for b in list(self.block_key):                  # a cached block still in use
            if self.ref[b] > 0:
                del self.cache[self.block_key.pop(b)]
                return b
        return self.free.pop()

    monkeypatch.setattr(oalloc.Allocator, "_take", greedy_take)
    with pytest.raises(AssertionError):
        run()


def test_utilisation_readout():
    a = Allocator(10, 4)
    a.add_seq_tokens(1, list(range(10)))       # 3 blocks, 10 slots filled
    a.add_seq(2, 1)                             # 1 block, 1 slot
    assert a.stats()["filled_slots"] == 11 and a.stats()["used_blocks"] == 4
    assert a.utilisation() == pytest.approx(11 / 16)
    a.fork(1, 3)                                # shared blocks count once
    assert a.utilisation() == pytest.approx(11 / 16)
