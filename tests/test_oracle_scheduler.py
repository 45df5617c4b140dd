"""The oracle's continuous-batching scheduler against the pages and against
independent formulations: the slot-simulation results the Ultralytics page
prints, a tick-by-tick slot simulation written here, and a token-label replay
that follows every cached token through swap-out and swap-in."""
import json
import os
import random

import pytest
from hypothesis import given, settings, strategies as st

from oracle import pkv_oracle as O
from oracle import scheduler as SC

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_worked_numbers.json")))


def run(sched):
    steps = []
    while True:
        s = sched.step()
        if not s.prefill and not s.decode:
            return steps
        steps.append(s)


def make(outputs, slots, policy, prompts=None, num_blocks=100000, tokens=100000, host=0):
    sched = SC.SchedulerModel(O.BlockAllocatorModel(num_blocks), slots, tokens, policy, host)
    for i, n in enumerate(outputs):
        sched.add_request(1 if prompts is None else prompts[i], n)
    return sched


@pytest.mark.parametrize("policy,steps_key,busy_key", [(SC.STATIC, "static_steps", "static_busy"),
                                                        (SC.CONTINUOUS, "continuous_steps", "continuous_busy")])
def test_slot_simulation_of_the_page(policy, steps_key, busy_key):
    g = GOLDEN["slot_simulation"]
    sched = make(g["lengths"], g["slots"], policy)
    run(sched)
    assert sched.steps == g[steps_key]
    assert round(sched.busy / (sched.steps * g["slots"]), 2) == g[busy_key]
    assert sched.busy == sum(g["lengths"])


def tick_simulation(outputs, slots, static):
    """Independent formulation: every tick each occupied slot produces a token;
    an empty slot takes the next request (static: only when all are empty)."""
    remaining = [0] * slots
    queue = list(outputs)
    ticks = 0
    while queue or any(remaining):
        if not static or not any(remaining):
            for k in range(slots):
                if remaining[k] == 0 and queue:
                    remaining[k] = queue.pop(0)
        remaining = [max(0, x - 1) for x in remaining]
        ticks += 1
    return ticks


@settings(max_examples=60, deadline=None)
@given(st.lists(st.integers(1, 40), min_size=1, max_size=25), st.integers(1, 6), st.booleans())
def test_steps_equal_a_tick_by_tick_slot_simulation(outputs, slots, static):
    sched = make(outputs, slots, SC.STATIC if static else SC.CONTINUOUS)
    run(sched)
    assert sched.steps == tick_simulation(outputs, slots, static)


def replay_labels(sched, steps_fn):
    """Apply every step's copies and writes to a pool of token labels and check
    that each running request's table gathers its tokens 0..len-1 in order."""
    alloc = sched.alloc
    P = alloc.block_size
    dev = {}           # (block, offset) -> (rid, pos)
    host = {}
    n_steps = 0
    while True:
        s = sched.step()
        if not s.prefill and not s.decode:
            break
        n_steps += 1
        # swap-out copies read the device blocks before this step writes anything
        for d, h in s.swap_out_pairs:
            for o in range(P):
                host[(h, o)] = dev.get((d, o))
        for h, d in s.swap_in_pairs:
            for o in range(P):
                dev[(d, o)] = host.get((h, o))
        labels = []
        for rid, n in zip(s.prefill, s.prefill_lens):
            labels += [(rid, p) for p in range(n)]
        for rid in s.decode:
            r = sched.requests[rid]
            labels.append((rid, alloc.num_tokens(r.seq) - 1))
        assert len(labels) == len(s.slots) == len(set(s.slots))
        for slot, lab in zip(s.slots, labels):
            dev[(slot // P, slot % P)] = lab
        for r in sched.running:
            t = alloc.block_table(r.seq)
            n = alloc.num_tokens(r.seq)
            got = [dev.get((t[p // P], p % P)) for p in range(n)]
            assert got == [(r.rid, p) for p in range(n)], r.rid
        steps_fn(s)
    return n_steps


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 10**6))
def test_memory_pressure_with_swapping_keeps_every_token_and_finishes_every_request(seed):
    rnd = random.Random(seed)
    nb = rnd.randint(8, 40)
    max_seqs = rnd.randint(1, 8)
    tokens = rnd.randint(32, 200)
    sched = SC.SchedulerModel(O.BlockAllocatorModel(nb, 16, rnd.sample(range(nb), nb)), max_seqs, tokens,
                              rnd.choice([SC.CONTINUOUS, SC.STATIC]), num_host_blocks=4 * nb)
    outputs = []
    for _ in range(rnd.randint(1, 15)):
        while True:
            p, o = rnd.randint(1, min(tokens, 60)), rnd.randint(1, 80)
            if -(-(p + o) // 16) <= nb:
                break
        sched.add_request(p, o)
        outputs.append(o)

    def check(s):
        a = sched.alloc
        assert len(sched.running) <= max_seqs
        assert sum(s.prefill_lens) + len(s.decode) <= tokens
        used = set()
        for r in sched.running:
            t = a.block_table(r.seq)
            assert len(t) == -(-a.num_tokens(r.seq) // 16)
            used |= set(t)
        assert a.num_free + len(used) == nb
        assert len(sched.host_free) + sum(len(r.host_table) for r in sched.swapped) == 4 * nb

    replay_labels(sched, check)
    assert sched.done()
    assert [r.generated for r in sched.requests] == outputs
    assert sched.busy == sum(outputs)
    assert sched.alloc.num_free == nb


def test_a_full_pool_swaps_out_the_newest_request_and_brings_it_back():
    # 4 blocks; two requests of 31 tokens (2 blocks) grow until the pool is full
    sched = SC.SchedulerModel(O.BlockAllocatorModel(4), 4, 1000, SC.CONTINUOUS, num_host_blocks=8)
    sched.add_request(31, 20)
    sched.add_request(31, 20)
    s0 = sched.step()
    assert s0.prefill == [0, 1] and s0.decode == []
    s1 = sched.step()                 # both decode: token 31 fits their second block
    assert s1.decode == [0, 1] and not s1.swapped_out
    table1 = sched.alloc.block_table(sched.requests[1].seq)
    s2 = sched.step()                 # request 0 needs a third block: request 1 goes out
    assert s2.swapped_out == [1] and s2.decode == [0]
    assert [d for d, _ in s2.swap_out_pairs] == table1
    assert [h for _, h in s2.swap_out_pairs] == [0, 1]      # host blocks first in first out
    steps = run(sched)
    back = [s for s in steps if s.swapped_in]
    assert back and back[0].swapped_in == [1]
    assert all(r.generated == 20 for r in sched.requests)


def test_requests_that_can_never_fit_are_rejected():
    sched = SC.SchedulerModel(O.BlockAllocatorModel(4), 2, 64, SC.CONTINUOUS)
    with pytest.raises(ValueError):
        sched.add_request(65, 1)           # over the token budget
    with pytest.raises(ValueError):
        sched.add_request(40, 40)          # 80 tokens > 4 blocks
    with pytest.raises(ValueError):
        sched.add_request(0, 5)
