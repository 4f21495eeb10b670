"""Host block allocator model: free list, reference counts, copy-on-write.

Rules, each from the pages:

* The pool is a list of equal-size physical blocks; a free list hands them
  out with ``pop()`` from its end and takes them back with ``append``
  (KV Cache从原理到实战 §6.2, the paged sketch).  Asking for more blocks than
  are free fails before anything is taken ("Out of KV cache blocks"), so a
  failed request changes nothing.
* A sequence's block table lists its physical blocks in logical order; a new
  physical block is taken only when every earlier block is full, so a
  sequence wastes less than one block (KV 缓存与分页注意力 §07; Paged
  Attention in LLMs, "Paged Attention 如何工作").
* Parallel samples of one prompt point at the same physical blocks, and each
  block counts how many sequences use it.  Before a sequence writes into a
  block that others still use, the block is copied to a fresh one, the write
  goes into the copy, and the original's count drops by one (KV 缓存与分页
  注意力 §08).  Reading: the writer copies while the count is above one; the
  last holder writes in place.
* A finished sequence gives its blocks back (§07); a block returns to the
  free list when its count reaches zero.  Blocks go back in table order.
* A logical index past the table is an index error (KV Cache内存优化技术原理与
  PagedAttention分页注意力实现, the BlockTable sketch).

Prefix caching (KV 缓存与分页注意力 §11 后来的做法; KV Cache从原理到实战 §4.2):

* Every full block of a sequence whose token ids are known is identified by
  its tokens and everything before them.  Here that identity is written out
  plainly: the tuple of all token ids from the sequence's start to the end
  of the block.  A new sequence whose first blocks have identities already
  held reuses those blocks (longest matching run of full blocks from the
  start; the first miss ends it) and takes fresh blocks for the rest; a
  block with the same tokens after a different beginning is not the same
  block (the same word at another position has other keys and values, §12).
* Reused blocks are reference-counted like shared prompt blocks; a block
  whose count reaches zero but whose identity is held stays cached (its
  contents kept) in a least-recently-used list, and is taken back, or
  reused by a later match, from there.  Readings: a fresh block comes from
  the free list first and only then from the LRU end of the cached list
  (never a referenced block, §4.2); a finished sequence's cached blocks
  join the list last block first, so a sequence's later blocks are evicted
  before its earlier ones; when an identity is already held by another
  block, the new block stays unregistered.
* Utilisation (§05, §07): token slots holding a token over the slots of the
  blocks in use.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


class OutOfBlocks(RuntimeError):
    pass


class UnknownSequence(KeyError):
    pass


class RefcountError(RuntimeError):
    pass


class Allocator:
    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        if free_order is None:
            self.free: List[int] = list(range(num_blocks))
        else:
            fo = [int(b) for b in free_order]
            if sorted(fo) != list(range(num_blocks)):
                raise ValueError("free_order must be a permutation of the pool")
            self.free = fo
        self.ref = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        # prefix caching: token ids of sequences admitted with them (None: not known),
        # identity -> block, block -> identity, and cached unreferenced blocks (LRU first)
        self.tokens: Dict[int, Optional[List[int]]] = {}
        self.cache: Dict[tuple, int] = {}
        self.block_key: Dict[int, tuple] = {}
        self.evictable: List[int] = []
        self.hit_blocks = 0
        self.evictions = 0

    # -- helpers
    def _need(self, n_tokens: int) -> int:
        return (n_tokens + self.block_size - 1) // self.block_size

    def _seq(self, seq_id: int) -> List[int]:
        if seq_id not in self.tables:
            raise UnknownSequence(seq_id)
        return self.tables[seq_id]

    def available(self) -> int:
        """Blocks a request may take: free ones and cached unreferenced ones."""
        return len(self.free) + len(self.evictable)

    def _take(self) -> int:
        """A fresh block: from the free list, else the least recently used cached one."""
        if self.free:
            return self.free.pop()
        b = self.evictable.pop(0)
        del self.cache[self.block_key.pop(b)]
        self.evictions += 1
        return b

    def _identity(self, tokens: List[int], j: int) -> tuple:
        """Identity of full block j of a sequence: its tokens and everything before."""
        return tuple(tokens[:(j + 1) * self.block_size])

    def _register(self, table: List[int], tokens: List[int], j: int) -> None:
        """Make full block j of a sequence findable by its identity (if not held)."""
        key = self._identity(tokens, j)
        b = table[j]
        if key not in self.cache and b not in self.block_key:
            self.cache[key] = b
            self.block_key[b] = key

    # -- operations
    def add_seq(self, seq_id: int, num_tokens: int) -> List[int]:
        if seq_id in self.tables:
            raise ValueError(f"sequence {seq_id} exists")
        if num_tokens < 0:
            raise ValueError("negative length")
        need = self._need(num_tokens)
        if need > self.available():
            raise OutOfBlocks("Out of KV cache blocks")
        blocks = [self._take() for _ in range(need)]
        for b in blocks:
            self.ref[b] = 1
        self.tables[seq_id] = blocks
        self.lens[seq_id] = num_tokens
        self.tokens[seq_id] = None
        return list(blocks)

    def add_seq_tokens(self, seq_id: int, tokens: Sequence[int]) -> int:
        """New sequence with known token ids, reusing cached blocks of the same
        beginning; returns how many of its tokens are already cached."""
        if seq_id in self.tables:
            raise ValueError(f"sequence {seq_id} exists")
        tokens = [int(t) for t in tokens]
        n, bs = len(tokens), self.block_size
        matched = []
        for j in range(n // bs):
            b = self.cache.get(self._identity(tokens, j))
            if b is None:
                break
            matched.append(b)
        need = self._need(n) - len(matched)
        reclaimed = sum(1 for b in matched if self.ref[b] == 0)
        if need > self.available() - reclaimed:
            raise OutOfBlocks("Out of KV cache blocks")
        for b in matched:
            if self.ref[b] == 0:
                self.evictable.remove(b)
            self.ref[b] += 1
        self.hit_blocks += len(matched)
        table = list(matched)
        for _ in range(need):
            b = self._take()
            self.ref[b] = 1
            table.append(b)
        for j in range(len(matched), n // bs):
            self._register(table, tokens, j)
        self.tables[seq_id] = table
        self.lens[seq_id] = n
        self.tokens[seq_id] = tokens
        return len(matched) * bs

    def fork(self, parent_id: int, child_id: int) -> None:
        table = self._seq(parent_id)
        if child_id in self.tables:
            raise ValueError(f"sequence {child_id} exists")
        self.tables[child_id] = list(table)
        self.lens[child_id] = self.lens[parent_id]
        toks = self.tokens.get(parent_id)
        self.tokens[child_id] = None if toks is None else list(toks)
        for b in table:
            self.ref[b] += 1

    def append_slots(self, seq_ids: Sequence[int],
                     token_ids: Optional[Sequence[int]] = None) -> Tuple[List[int], List[Tuple[int, int]]]:
        """One new token for each sequence; returns (slots, copy-on-write pairs).
        With ``token_ids`` a block filled by its last token becomes findable by
        later sequences; without them a sequence's tokens are no longer known."""
        ids = [int(s) for s in seq_ids]
        if token_ids is not None and len(token_ids) != len(ids):
            raise ValueError("one token id per sequence")
        if len(set(ids)) != len(ids):
            raise ValueError("duplicate sequence in one append")
        for s in ids:
            self._seq(s)
        # count blocks first so that a shortage changes nothing
        need, pending = 0, {}
        for s in ids:
            n, table = self.lens[s], self.tables[s]
            if n % self.block_size == 0:
                need += 1
            else:
                last = table[-1]
                if self.ref[last] - pending.get(last, 0) > 1:
                    need += 1
                    pending[last] = pending.get(last, 0) + 1
        if need > self.available():
            raise OutOfBlocks("Out of KV cache blocks")
        slots, pairs = [], []
        for i, s in enumerate(ids):
            n, table = self.lens[s], self.tables[s]
            if n % self.block_size == 0:              # previous blocks full: new block
                b = self._take()
                self.ref[b] = 1
                table.append(b)
            else:
                last = table[-1]
                if self.ref[last] > 1:                # shared: copy on write
                    b = self._take()
                    self.ref[last] -= 1
                    self.ref[b] = 1
                    table[-1] = b
                    pairs.append((last, b))
            slots.append(table[n // self.block_size] * self.block_size + n % self.block_size)
            self.lens[s] = n + 1
            toks = self.tokens.get(s)
            if token_ids is None or toks is None:
                self.tokens[s] = None
            else:
                toks.append(int(token_ids[i]))
                if (n + 1) % self.block_size == 0:    # the block is full now
                    self._register(table, toks, n // self.block_size)
        return slots, pairs

    def free_seq(self, seq_id: int) -> None:
        table = self._seq(seq_id)
        for b in table:
            if self.ref[b] <= 0:
                raise RefcountError(f"block {b} has no references")
        for b in table:
            self.ref[b] -= 1
        for b in table:                               # uncached blocks: free list, table order
            if self.ref[b] == 0 and b not in self.block_key:
                self.free.append(b)
        for b in reversed(table):                     # cached ones: LRU list, last block first
            if self.ref[b] == 0 and b in self.block_key:
                self.evictable.append(b)
        del self.tables[seq_id]
        del self.lens[seq_id]
        self.tokens.pop(seq_id, None)

    # -- swapping (KV 缓存与分页注意力 §09 放不下的时候): a preempted sequence's blocks
    # are all moved to CPU memory or none are, and all come back together
    def swap_out(self, seq_id: int, cpu: "Allocator") -> List[Tuple[int, int]]:
        """Move a sequence to ``cpu`` (an allocator over host blocks): it gets fresh
        host blocks in the same logical order and gives up its device blocks.
        Returns the (device block, host block) copies to make before the device
        blocks are reused.  Nothing changes if the host pool is short."""
        table = self._seq(seq_id)
        if seq_id in cpu.tables:
            raise ValueError(f"sequence {seq_id} exists on the host")
        host = cpu.add_seq(seq_id, self.lens[seq_id])
        pairs = list(zip(table, host))
        self.free_seq(seq_id)
        return pairs

    def swap_in(self, seq_id: int, cpu: "Allocator") -> List[Tuple[int, int]]:
        """Bring a swapped-out sequence back: fresh device blocks in the same logical
        order; returns the (host block, device block) copies to make before the
        sequence is read.  Nothing changes if the device pool is short."""
        host = cpu._seq(seq_id)
        if seq_id in self.tables:
            raise ValueError(f"sequence {seq_id} exists on the device")
        dev = self.add_seq(seq_id, cpu.lens[seq_id])
        pairs = list(zip(host, dev))
        cpu.free_seq(seq_id)
        return pairs

    def physical_block(self, seq_id: int, logical_idx: int) -> int:
        table = self._seq(seq_id)
        if logical_idx < 0 or logical_idx >= len(table):
            raise IndexError(f"logical block {logical_idx} out of range")
        return table[logical_idx]

    def slot(self, seq_id: int, pos: int) -> int:
        self._seq(seq_id)
        if pos < 0 or pos >= self.lens[seq_id]:
            raise IndexError(f"token {pos} out of range")
        return self.physical_block(seq_id, pos // self.block_size) * self.block_size \
            + pos % self.block_size

    def export(self, seq_ids: Sequence[int], max_blocks: int):
        """Block tables int32 [n, max_blocks] (-1 padded) and context lengths int32 [n]."""
        tables = np.full((len(seq_ids), max_blocks), -1, dtype=np.int32)
        lens = np.zeros(len(seq_ids), dtype=np.int32)
        for i, s in enumerate(seq_ids):
            table = self._seq(int(s))
            if len(table) > max_blocks:
                raise IndexError("table longer than max_blocks")
            tables[i, :len(table)] = table
            lens[i] = self.lens[int(s)]
        return tables, lens

    def num_free(self) -> int:
        return len(self.free)

    def num_evictable(self) -> int:
        return len(self.evictable)

    def stats(self) -> Dict[str, int]:
        """Block counts and the token slots in use (each used block once)."""
        bs = self.block_size
        fill: Dict[int, int] = {}
        for s, table in self.tables.items():
            n = self.lens[s]
            for k, b in enumerate(table):
                fill[b] = max(fill.get(b, 0), min(bs, max(0, n - k * bs)))
        used = sum(1 for r in self.ref if r > 0)
        return {"num_blocks": self.num_blocks, "free_blocks": len(self.free),
                "evictable_blocks": len(self.evictable), "used_blocks": used,
                "cached_blocks": len(self.block_key), "filled_slots": sum(fill.values()),
                "prefix_hit_blocks": self.hit_blocks, "evictions": self.evictions}

    def utilisation(self) -> float:
        """Token slots holding a token / token slots of the blocks in use."""
        st = self.stats()
        return st["filled_slots"] / (st["used_blocks"] * self.block_size) if st["used_blocks"] else 1.0

    def refcount(self, block: int) -> int:
        return self.ref[block]
