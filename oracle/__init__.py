"""CPU oracle for paged decode attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the
HIP library and its Python binding) never imports, links or calls it, and
this package imports nothing from the product.

What it computes is the plain definition, in float64, written from the pages:

* decode attention: the new token's query is dotted with every cached key,
  the scores are turned into weights, and the weighted sum of the cached
  values is the head's output (KV Cache从原理到实战 §2.1; KV 缓存与分页注意力
  §02).  Paging changes where K/V live, not what is computed: the kernel
  fetches K/V block by block through the block table (KV 缓存与分页注意力
  §07), so the oracle first gathers each sequence's tokens through its block
  table into contiguous arrays and then applies the textbook formula.
* multi-token attention for the prompt phase and chunked prefill: each new
  token's query attends over the cached tokens up to and including its own
  position (KV 缓存与分页注意力 §02; KV Cache从原理到实战 §2.3, §5.4);
* the cache write, the copy-on-write block copy, the host block allocator
  (free list, reference counts, copy-on-write; KV 缓存与分页注意力 §07–§08,
  KV Cache从原理到实战 §6.2), the per-token KV size (§03 / §2.2), and the
  8-bit float format used for an fp8 cache (KV 缓存与分页注意力 §11).

Every function is pinned by tests under ``tests/`` against things other than
itself: values printed on the pages, brute force, closed forms, invariants and
library routines.  Nothing here is "parity unpinned".
"""
from .formats import (decode, e4m3_decode_table, e4m3_encode, e4m3_values,  # noqa: F401
                      int8_group_encode)
from .attention import (gather_sequence, paged_attention, contiguous_attention,  # noqa: F401
                        partition_states, lse_combine, kv_write, kv_write_int8, copy_blocks,
                        swap_blocks)
from .prefill import paged_prefill, query_positions  # noqa: F401
from .allocator import Allocator, OutOfBlocks, UnknownSequence, RefcountError  # noqa: F401
from .sizes import kv_bytes_per_token  # noqa: F401
