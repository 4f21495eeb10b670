"""Multi-token paged attention (prompt phase / chunked prefill) — plain float64 definition.

TEST INFRASTRUCTURE ONLY (see the package header).

Generation has two phases: the prompt phase handles a whole prompt at once
and produces every prompt token's key and value together; the generation
phase then adds one token per round (KV 缓存与分页注意力 §02 一次写一个词元).
The prompt phase is compute-bound, the generation phase bandwidth-bound
(KV Cache从原理到实战 §2.3), and a long prompt can be cut into chunks so
that its prefill does not block decoding (§5.4, chunked prefill).

What one call computes, for a batch of sequences: sequence s holds
``n = context_lens[s]`` tokens in the paged cache, its last ``q_len`` of them
being the chunk just written (``q_len = query_start[s+1] - query_start[s]``).
Query row ``r = query_start[s] + i`` (i < q_len) belongs to the token at
position ``p = n - q_len + i``; like the one new token of a decode step, it
attends over every cached token up to and including itself, and none after
it (a causal mask over the new tokens; the tokens before the chunk are all
visible).  So each query row's output is exactly the decode definition over
the first ``p + 1`` tokens of its sequence.  Reading taken where the pages
are silent: a row with ``p < 0`` (a chunk longer than its context) has
nothing to attend to and gives zeros.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

from .attention import _attend_one, gather_sequence
from .formats import decode


def query_positions(n: int, q_len: int) -> np.ndarray:
    """Positions of a sequence's q_len query rows: the last q_len of its n tokens."""
    return n - q_len + np.arange(q_len)


def paged_prefill(q: np.ndarray, q_dtype: str, k_pool: np.ndarray, v_pool: np.ndarray,
                  kv_dtype: str, block_tables: np.ndarray, context_lens: Sequence[int],
                  query_start: Sequence[int], block_size: int, scale: float,
                  k_scale: float = 1.0, v_scale: float = 1.0,
                  rows: Sequence[int] = None) -> np.ndarray:
    """Causal multi-token attention over a paged cache, float64 [T, H, D].

    ``q`` is [T, H, D] with the rows of sequence s at
    ``query_start[s]:query_start[s+1]``.  For each row: gather the sequence's
    tokens through its block table, keep those at positions <= the row's own
    position, and apply the decode definition (softmax of the scaled dot
    products, weighted sum of values; heads share KV groups as in decode).
    ``rows`` restricts the work to some query rows (others stay zero).
    """
    Q = decode(q, q_dtype)
    T, H, D = Q.shape
    out = np.zeros((T, H, D), dtype=np.float64)
    qs = np.asarray(query_start, dtype=np.int64)
    wanted = None if rows is None else set(int(r) for r in rows)
    for s in range(len(qs) - 1):
        r0, r1 = int(qs[s]), int(qs[s + 1])
        n = int(context_lens[s])
        if r1 <= r0 or n <= 0:
            continue
        if wanted is not None and not any(r in wanted for r in range(r0, r1)):
            continue
        K = gather_sequence(k_pool, kv_dtype, block_tables[s], n, block_size, k_scale)
        V = gather_sequence(v_pool, kv_dtype, block_tables[s], n, block_size, v_scale)
        for i, p in enumerate(query_positions(n, r1 - r0)):
            if p < 0 or (wanted is not None and r0 + i not in wanted):
                continue
            out[r0 + i] = _attend_one(Q[r0 + i], K[:p + 1], V[:p + 1], scale)
    return out
