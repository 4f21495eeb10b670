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

    # -- helpers
    def _need(self, n_tokens: int) -> int:
        return (n_tokens + self.block_size - 1) // self.block_size

    def _seq(self, seq_id: int) -> List[int]:
        if seq_id not in self.tables:
            raise UnknownSequence(seq_id)
        return self.tables[seq_id]

    # -- operations
    def add_seq(self, seq_id: int, num_tokens: int) -> List[int]:
        if seq_id in self.tables:
            raise ValueError(f"sequence {seq_id} exists")
        if num_tokens < 0:
            raise ValueError("negative length")
        need = self._need(num_tokens)
        if need > len(self.free):
            raise OutOfBlocks("Out of KV cache blocks")
        blocks = [self.free.pop() for _ in range(need)]
        for b in blocks:
            self.ref[b] = 1
        self.tables[seq_id] = blocks
        self.lens[seq_id] = num_tokens
        return list(blocks)

    def fork(self, parent_id: int, child_id: int) -> None:
        table = self._seq(parent_id)
        if child_id in self.tables:
            raise ValueError(f"sequence {child_id} exists")
        self.tables[child_id] = list(table)
        self.lens[child_id] = self.lens[parent_id]
        for b in table:
            self.ref[b] += 1

    def append_slots(self, seq_ids: Sequence[int]) -> Tuple[List[int], List[Tuple[int, int]]]:
        """One new token for each sequence; returns (slots, copy-on-write pairs)."""
        ids = [int(s) for s in seq_ids]
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
        if need > len(self.free):
            raise OutOfBlocks("Out of KV cache blocks")
        slots, pairs = [], []
        for s in ids:
            n, table = self.lens[s], self.tables[s]
            if n % self.block_size == 0:              # previous blocks full: new block
                b = self.free.pop()
                self.ref[b] = 1
                table.append(b)
            else:
                last = table[-1]
                if self.ref[last] > 1:                # shared: copy on write
                    b = self.free.pop()
                    self.ref[last] -= 1
                    self.ref[b] = 1
                    table[-1] = b
                    pairs.append((last, b))
            slots.append(table[n // self.block_size] * self.block_size + n % self.block_size)
            self.lens[s] = n + 1
        return slots, pairs

    def free_seq(self, seq_id: int) -> None:
        table = self._seq(seq_id)
        for b in table:
            if self.ref[b] <= 0:
                raise RefcountError(f"block {b} has no references")
        for b in table:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.tables[seq_id]
        del self.lens[seq_id]

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

    def refcount(self, block: int) -> int:
        return self.ref[block]
