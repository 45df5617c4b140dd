"""Pins of the oracle's block-allocator model: closed forms and invariants.

The model's policy (FIFO free list, copy of a partially filled shared last
block) is a reading; what the pages fix is checked here independently of it:
ceil(len / 16) blocks per sequence, waste only in the last block, refcounts equal
to the number of tables holding a block, every block either free or referenced,
copy-on-write only for a shared block with room, atomic failure when the pool is
short, and the block counts of the parallel-sampling workload.
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import pkv_oracle as O
from pkv_workloads import parallel_sampling

P = 16


def _invariants(a: O.BlockAllocatorModel):
    held = {}
    for sid, table in a.tables.items():
        n = a.lens[sid]
        assert len(table) == -(-n // P), "a sequence holds ceil(len / 16) blocks"
        assert len(set(table)) == len(table)
        for b in table:
            held[b] = held.get(b, 0) + 1
    for b in range(a.num_blocks):
        assert a.refcount(b) == held.get(b, 0), "refcount = number of tables holding the block"
    assert set(a.free).isdisjoint(held), "a free block is never referenced"
    assert len(a.free) + len(held) == a.num_blocks, "every block is free or referenced"
    assert len(set(a.free)) == len(a.free)


@pytest.mark.parametrize("n", [1, 5, 15, 16, 17, 31, 32, 33, 200, 2000])
def test_fresh_sequence_gets_ceil_blocks_and_consecutive_slots(n):
    a = O.BlockAllocatorModel(200, P)
    s = a.create()
    slots, pairs = a.append_slots(s, n)
    t = a.block_table(s)
    assert pairs == []
    assert len(t) == math.ceil(n / P)
    assert slots == [t[i // P] * P + i % P for i in range(n)]
    # the only unused reserved slots are in the last block, fewer than one block
    assert 0 <= len(t) * P - n < P
    _invariants(a)


def test_blocks_come_first_in_first_out_and_return_to_the_back():
    order = [5, 2, 7, 0, 1, 3, 6, 4]
    a = O.BlockAllocatorModel(8, P, order)
    s0, s1 = a.create(), a.create()
    a.append_slots(s0, 33)            # takes 5, 2, 7
    a.append_slots(s1, 1)             # takes 0
    assert a.block_table(s0) == [5, 2, 7] and a.block_table(s1) == [0]
    a.free_seq(s0)
    assert list(a.free) == [1, 3, 6, 4, 5, 2, 7]
    s2 = a.create()
    a.append_slots(s2, 20)
    assert a.block_table(s2) == [1, 3]
    _invariants(a)


def test_one_token_at_a_time_allocates_only_when_the_last_block_is_full():
    a = O.BlockAllocatorModel(10, P)
    s = a.create()
    for i in range(50):
        before = a.num_free
        slots, _ = a.append_slots(s, 1)
        assert (before - a.num_free) == (1 if i % P == 0 else 0)
        assert slots[0] == a.block_table(s)[-1] * P + i % P


def test_fork_shares_every_block_and_partial_shared_block_is_copied_once_per_writer():
    a = O.BlockAllocatorModel(40, P)
    root = a.create()
    a.append_slots(root, 40)                      # 2 full blocks + 8 tokens
    kids = [a.fork(root) for _ in range(3)]
    shared = a.block_table(root)
    for b in shared:
        assert a.refcount(b) == 4
    pairs_seen = []
    for i, s in enumerate([root] + kids):
        slots, pairs = a.append_slots(s, 1)
        t = a.block_table(s)
        assert t[:2] == shared[:2], "full shared blocks stay shared"
        if i < 3:
            assert pairs == [(shared[2], t[2])] and t[2] != shared[2]
            pairs_seen.append(pairs[0])
        else:
            assert pairs == [] and t[2] == shared[2], "the last holder writes in place"
        assert slots == [t[2] * P + 8]
    assert a.refcount(shared[2]) == 1
    assert len({d for _, d in pairs_seen}) == 3
    _invariants(a)


def test_full_shared_last_block_is_not_copied():
    a = O.BlockAllocatorModel(10, P)
    root = a.create()
    a.append_slots(root, 32)
    kid = a.fork(root)
    slots, pairs = a.append_slots(kid, 1)
    assert pairs == []
    t = a.block_table(kid)
    assert t[:2] == a.block_table(root) and len(t) == 3 and slots == [t[2] * P]
    _invariants(a)


def test_out_of_blocks_changes_nothing():
    a = O.BlockAllocatorModel(4, P, [3, 1, 0, 2])
    s = a.create()
    a.append_slots(s, 40)
    k = a.fork(s)
    snap = (list(a.free), list(a.ref), {i: list(t) for i, t in a.tables.items()}, dict(a.lens))
    with pytest.raises(O.OutOfBlocks):
        a.append_slots(k, 30)            # needs a copy + 2 blocks, only 1 free
    assert snap == (list(a.free), list(a.ref), {i: list(t) for i, t in a.tables.items()}, dict(a.lens))
    slots, pairs = a.append_slots(k, 8)   # copy only: fits
    assert len(pairs) == 1 and a.num_free == 0
    _invariants(a)


def test_unknown_sequence_is_rejected():
    a = O.BlockAllocatorModel(4, P)
    s = a.create()
    a.free_seq(s)
    with pytest.raises(O.UnknownSequence):
        a.append_slots(s, 1)
    with pytest.raises(O.UnknownSequence):
        a.fork(s)
    with pytest.raises(O.UnknownSequence):
        a.free_seq(s)


def test_parallel_sampling_block_counts_match_the_closed_form():
    w = parallel_sampling(seed=4, groups=3, samples=8, with_rows=False)
    a = O.BlockAllocatorModel(w.num_blocks, P, w.initial_free_order)
    n_pairs = 0
    for op in w.ops:
        if op[0] == "create":
            a.create()
        elif op[0] == "fork":
            a.fork(op[1])
        elif op[0] == "append":
            n_pairs += len(a.append_slots(op[1], op[2])[1])
    _invariants(a)
    tails = w.tails
    used = w.num_blocks - a.num_free
    # 62 full prompt blocks shared by all 8 samples + each sample's own tail pages
    # (its 8 prompt tokens of the partial block plus its tail)
    assert used == sum(62 + sum(math.ceil((8 + int(t)) / P) for t in tails[g]) for g in range(3))
    assert n_pairs == 3 * 7
    shared = [b for b in range(w.num_blocks) if a.refcount(b) == 8]
    assert len(shared) == 3 * 62
    # saving versus unshared copies: 7 extra copies of 62 prompt blocks per group
    unshared = sum(math.ceil((1000 + int(t)) / P) for t in tails.ravel())
    assert unshared - used == 3 * 7 * 62


@settings(max_examples=150, deadline=None)
@given(st.lists(st.tuples(st.integers(0, 3), st.integers(0, 9), st.integers(0, 40)), min_size=1, max_size=60))
def test_random_operation_sequences_keep_the_invariants(ops):
    a = O.BlockAllocatorModel(24, P, list(np.random.default_rng(0).permutation(24)))
    live = []
    for kind, pick, n in ops:
        if kind == 0 or not live:
            live.append(a.create())
        elif kind == 1:
            s = live[pick % len(live)]
            try:
                slots, pairs = a.append_slots(s, n)
            except O.OutOfBlocks:
                continue
            t = a.block_table(s)
            L = a.num_tokens(s)
            assert slots == [t[i // P] * P + i % P for i in range(L - n, L)]
            for src, dst in pairs:
                assert a.refcount(dst) == 1
        elif kind == 2:
            live.append(a.fork(live[pick % len(live)]))
        else:
            a.free_seq(live.pop(pick % len(live)))
        _invariants(a)
    # no two live sequences own the same slot unless they share the block
    owner = {}
    for s in live:
        t = a.block_table(s)
        for i in range(a.num_tokens(s)):
            owner.setdefault(t[i // P] * P + i % P, set()).add(s)
    for slot, ss in owner.items():
        if len(ss) > 1:
            assert a.refcount(slot // P) >= len(ss)
