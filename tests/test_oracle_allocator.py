"""Pins for the oracle's allocator model and the per-token size closed form.

Worked examples and numbers printed on the pages live in
``tests/golden/pages_worked_examples.json`` (each entry cites its page and
section); invariants are checked on random operation sequences.
"""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import Allocator, OutOfBlocks, UnknownSequence, kv_bytes_per_token

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "pages_worked_examples.json"), encoding="utf-8"))
KB = 1024


# ------------------------------------------------------------------ closed forms
@pytest.mark.parametrize("row", GOLDEN["kv_bytes_per_token"], ids=lambda r: r["model"])
def test_kv_bytes_per_token_printed_values(row):
    b = kv_bytes_per_token(row["num_kv_heads"], row["head_dim"], row["num_layers"], row["dtype_bytes"])
    assert b == row["bytes"]
    if "per_layer_bytes" in row:
        assert kv_bytes_per_token(row["num_kv_heads"], row["head_dim"], 1, row["dtype_bytes"]) \
            == row["per_layer_bytes"]


def test_size_ratio_and_sizing_printed_values():
    per = {r["model"]: r["bytes"] for r in GOLDEN["kv_bytes_per_token"]}
    assert per["Llama-2-70B"] / per["OPT-13B"] == GOLDEN["ratio_llama70b_to_opt13b"]["value"]
    s = {r["what"]: r for r in GOLDEN["sizing"]}
    opt = per["OPT-13B"]
    assert abs(2048 * opt / (KB * KB * KB) - s["one OPT-13B sequence at 2,048 tokens"]["approx_gb"]) < 0.05
    tokens = 12 * 2 ** 30 // opt
    assert abs(tokens - s["tokens that fit in the 12 GB cache of a 40 GB A100"]["approx_tokens"]) < 50
    assert tokens // 2048 == s["sequences of 2,048 tokens that fit (reserve-max policy)"]["value"]
    llama = per["Llama-2-7B"]
    assert 4096 * 16 * llama == 32 * 2 ** 30
    assert 131072 * llama == 64 * 2 ** 30
    assert 2048 * llama == 1 * 2 ** 30


# ------------------------------------------------------------------ worked examples
def test_ten_tokens_block_size_four():
    ex = GOLDEN["paged_allocation_example"]
    a = Allocator(16, ex["block_size"])
    blocks = a.add_seq(1, ex["tokens"])
    assert len(blocks) == ex["blocks"]
    assert len(blocks) * ex["block_size"] - ex["tokens"] == ex["empty_slots_in_last_block"]
    assert ex["contiguous_reservation_slots"] - ex["tokens"] == ex["contiguous_waste"]
    # tokens arrive one by one: a new block only when the previous ones are full
    b = Allocator(16, ex["block_size"])
    b.add_seq(2, 0)
    sizes = []
    for _ in range(ex["tokens"]):
        b.append_slots([2])
        sizes.append(len(b.tables[2]))
    assert sizes == [1, 1, 1, 1, 2, 2, 2, 2, 3, 3]


def test_block_table_example_slots():
    ex = GOLDEN["block_table_example"]
    bs, table = ex["block_size"], ex["table"]
    n = 16
    free_order = [b for b in range(n) if b not in table] + list(reversed(table))
    a = Allocator(n, bs, free_order)
    a.add_seq(7, 10)
    assert a.tables[7] == table
    assert [a.physical_block(7, j) for j in range(3)] == table
    assert a.slot(7, 0) == 5 * 4 and a.slot(7, 9) == 3 * 4 + 1 and a.slot(7, 5) == 12 * 4 + 1
    with pytest.raises(IndexError):
        a.physical_block(7, 3)
    tables, lens = a.export([7], 4)
    assert tables.tolist() == [table + [-1]] and lens.tolist() == [10]


def test_copy_on_write_example():
    ex = GOLDEN["copy_on_write_example"]
    bs = ex["block_size"]
    prompt = (ex["shared_prompt_blocks"] - 1) * bs + ex["last_block_filled"]
    a = Allocator(8, bs)
    a.add_seq(0, prompt)
    a.fork(0, 1)
    last = a.tables[0][-1]
    assert a.refcount(last) == ex["refcount_before"]
    slots, pairs = a.append_slots([0])                   # first writer copies
    assert len(pairs) == 1 and pairs[0][0] == last
    new = pairs[0][1]
    assert a.refcount(last) == ex["refcount_after"] and a.refcount(new) == 1
    assert slots == [new * bs + ex["last_block_filled"]]
    assert a.tables[0][:-1] == a.tables[1][:-1]          # the full prompt block stays shared
    assert a.refcount(a.tables[0][0]) == 2
    slots2, pairs2 = a.append_slots([1])                 # last holder writes in place
    assert pairs2 == [] and slots2 == [last * bs + ex["last_block_filled"]]


def test_both_samples_in_one_append():
    a = Allocator(8, 4)
    a.add_seq(0, 6)
    a.fork(0, 1)
    last = a.tables[0][-1]
    slots, pairs = a.append_slots([0, 1])
    assert len(pairs) == 1 and a.tables[1][-1] == last and a.refcount(last) == 1


def test_full_shared_block_needs_no_copy():
    a = Allocator(8, 4)
    a.add_seq(0, 8)
    a.fork(0, 1)
    _, pairs = a.append_slots([0, 1])
    assert pairs == [] and a.tables[0][:2] == a.tables[1][:2]
    assert a.tables[0][2] != a.tables[1][2]


def test_out_of_blocks_is_atomic():
    a = Allocator(4, 4)
    a.add_seq(0, 9)                                      # 3 blocks
    with pytest.raises(OutOfBlocks):
        a.add_seq(1, 5)                                  # needs 2, 1 free
    assert a.num_free() == 1 and 1 not in a.tables
    a.add_seq(1, 4)
    a.fork(1, 2)
    free_before, tables_before = list(a.free), {k: list(v) for k, v in a.tables.items()}
    with pytest.raises(OutOfBlocks):
        a.append_slots([0, 1, 2])                        # 0 ok in place; 1 and 2 need new blocks
    assert a.free == free_before and a.tables == tables_before and a.lens[0] == 9


def test_errors():
    a = Allocator(4, 4)
    with pytest.raises(UnknownSequence):
        a.free_seq(3)
    with pytest.raises(UnknownSequence):
        a.append_slots([3])
    a.add_seq(0, 1)
    with pytest.raises(ValueError):
        a.add_seq(0, 1)
    with pytest.raises(ValueError):
        a.append_slots([0, 0])
    with pytest.raises(IndexError):
        a.export([0], 0)


def test_free_returns_blocks_lifo():
    a = Allocator(6, 2)
    a.add_seq(0, 5)                                      # pops 5, 4, 3
    assert a.tables[0] == [5, 4, 3]
    a.free_seq(0)
    assert a.free == [0, 1, 2, 5, 4, 3]
    a.add_seq(1, 2)
    assert a.tables[1] == [3]


# ------------------------------------------------------------------ invariants
def check_invariants(a: Allocator):
    counts = np.zeros(a.num_blocks, dtype=int)
    for s, t in a.tables.items():
        assert len(t) == math.ceil(a.lens[s] / a.block_size)     # waste < one block
        for b in t:
            counts[b] += 1
    assert counts.tolist() == a.ref
    assert len(set(a.free)) == len(a.free)
    assert all(a.ref[b] == 0 for b in a.free)
    assert len(a.free) + int((counts > 0).sum()) == a.num_blocks


ops = st.lists(st.tuples(st.sampled_from(["add", "fork", "append", "free"]),
                         st.integers(0, 7), st.integers(0, 7), st.integers(0, 13)),
               min_size=1, max_size=60)


@settings(max_examples=300, deadline=None)
@given(ops=ops, bs=st.sampled_from([1, 2, 4]), nb=st.integers(1, 24))
def test_random_operation_sequences_keep_invariants(ops, bs, nb):
    a = Allocator(nb, bs)
    for op, x, y, n in ops:
        try:
            if op == "add":
                a.add_seq(x, n)
            elif op == "fork":
                a.fork(x, y)
            elif op == "append":
                ids = sorted({x, y} & set(a.tables))
                before = {s: list(a.tables[s]) for s in ids}
                slots, pairs = a.append_slots(ids)
                for (src, dst) in pairs:
                    assert a.ref[dst] == 1 and a.ref[src] >= 1
                for s, slot in zip(ids, slots):
                    assert slot == a.slot(s, a.lens[s] - 1)
                    assert a.ref[slot // bs] == 1        # a write never lands in a shared block
            elif op == "free":
                a.free_seq(x)
        except (OutOfBlocks, UnknownSequence, ValueError):
            pass
        check_invariants(a)


# ------------------------------------------------------------------ swapping (§09)
def test_swap_out_and_in_keeps_contents_and_order():
    """A preempted sequence's blocks all go to the host and all come back (KV 缓存与
    分页注意力 §09); the data moves bit for bit and the logical order is kept, so
    the sequence reads back the same tokens from new physical blocks."""
    gpu, cpu = Allocator(12, 4), Allocator(6, 4)
    gpu.add_seq(1, 10)                        # 3 blocks
    gpu.add_seq(2, 5)
    rng = np.random.default_rng(0)
    dev = rng.integers(0, 255, size=(12, 4, 8), dtype=np.uint8)
    host = np.zeros((6, 4, 8), dtype=np.uint8)
    before = [dev[gpu.physical_block(1, k)].copy() for k in range(3)]
    pairs = gpu.swap_out(1, cpu)
    oracle.swap_blocks([host], [dev], pairs)
    assert 1 not in gpu.tables and cpu.lens[1] == 10 and gpu.num_free() == 12 - 2
    dev[[b for b, _ in pairs]] = 0            # the device blocks are reused by others
    back = gpu.swap_in(1, cpu)
    oracle.swap_blocks([dev], [host], back)
    assert cpu.num_free() == 6 and gpu.lens[1] == 10
    after = [dev[gpu.physical_block(1, k)] for k in range(3)]
    assert all(np.array_equal(x, y) for x, y in zip(before, after))


def test_swap_is_all_or_nothing():
    gpu, cpu = Allocator(8, 4), Allocator(2, 4)
    gpu.add_seq(1, 12)                        # 3 blocks, host has 2
    state = (list(gpu.free), list(gpu.ref), dict(gpu.lens))
    with pytest.raises(OutOfBlocks):
        gpu.swap_out(1, cpu)
    assert (list(gpu.free), list(gpu.ref), dict(gpu.lens)) == state and not cpu.tables
    gpu2 = Allocator(3, 4)
    cpu2 = Allocator(8, 4)
    gpu2.add_seq(1, 12)
    gpu2.swap_out(1, cpu2)
    gpu2.add_seq(2, 1)                        # the device pool is now short for 1
    with pytest.raises(OutOfBlocks):
        gpu2.swap_in(1, cpu2)
    assert 1 in cpu2.tables and 1 not in gpu2.tables


def test_swap_of_a_shared_sequence_keeps_the_sharer():
    """Swapping out one of two parallel samples leaves the other's blocks in place
    (counts drop by one); the swapped one gets its own copies."""
    gpu, cpu = Allocator(8, 4), Allocator(8, 4)
    gpu.add_seq(1, 6)
    gpu.fork(1, 2)
    shared = list(gpu.tables[1])
    pairs = gpu.swap_out(2, cpu)
    assert [g for g, _ in pairs] == shared and all(gpu.refcount(b) == 1 for b in shared)
    assert gpu.tables[1] == shared
