"""The native continuous-batching scheduler (pkv_scheduler_*) against the oracle
model, step by step and bit-exact: which requests finish, swap, prefill and
decode, every copy pair, every slot, and the block tables (no GPU needed)."""
import random

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import pkv_oracle as O
from oracle import scheduler as SC


@pytest.fixture(scope="module")
def PK():
    import paged_kv_cache_171_amd as PK
    return PK


def lockstep(PK, nb, order, max_seqs, tokens, policy, host, requests, bs=16):
    na = PK.BlockAllocator(nb, bs, order)
    ns = PK.Scheduler(na, max_seqs, tokens, policy, host)
    oa = O.BlockAllocatorModel(nb, bs, order)
    os_ = SC.SchedulerModel(oa, max_seqs, tokens, policy, host)
    for p, o in requests:
        assert ns.add_request(p, o) == os_.add_request(p, o)
    n = 0
    while True:
        s = ns.step()
        m = os_.step()
        assert list(s.finished) == m.finished
        assert list(s.swapped_out) == m.swapped_out
        assert [tuple(x) for x in s.swap_out_pairs] == m.swap_out_pairs
        assert list(s.swapped_in) == m.swapped_in
        assert [tuple(x) for x in s.swap_in_pairs] == m.swap_in_pairs
        assert list(s.prefill) == m.prefill
        assert list(np.diff(s.prefill_query_start_loc)) == m.prefill_lens
        assert list(s.decode) == m.decode
        assert list(s.slot_mapping) == m.slots
        assert na.num_free == oa.num_free
        for r in os_.running:
            state, seq, gen, ctx = ns.request(r.rid)
            assert state == PK.PKV_REQ_RUNNING and seq == r.seq and gen == r.generated
            t, length = na.seq_block_table(seq)
            assert t == oa.block_table(r.seq) and length == oa.num_tokens(r.seq) == ctx
        if s.empty:
            break
        n += 1
    steps, busy, waiting, running, swapped = ns.stats()
    assert (steps, busy) == (os_.steps, os_.busy) and (waiting, running, swapped) == (0, 0, 0)
    return n


def test_slot_simulation_of_the_page(PK):
    lengths = [5, 50, 8, 12, 40, 3, 30, 7]
    for policy, steps in ((PK.PKV_SCHED_CONTINUOUS, 50), (PK.PKV_SCHED_STATIC, 90)):
        assert lockstep(PK, 200, None, 4, 64, policy, 0, [(1, n) for n in lengths]) == steps


@settings(max_examples=60, deadline=None)
@given(st.integers(0, 10**6))
def test_random_workloads_under_memory_pressure_match_the_model(PK, seed):
    rnd = random.Random(seed)
    nb = rnd.randint(6, 48)
    bs = rnd.choice([8, 16, 16, 32])
    order = rnd.sample(range(nb), nb)
    tokens = rnd.randint(24, 160)
    reqs = []
    for _ in range(rnd.randint(1, 16)):
        while True:
            p, o = rnd.randint(1, min(tokens, 70)), rnd.randint(1, 90)
            if -(-(p + o) // bs) <= nb:
                break
        reqs.append((p, o))
    lockstep(PK, nb, order, rnd.randint(1, 9), tokens, rnd.choice([PK.PKV_SCHED_CONTINUOUS, PK.PKV_SCHED_STATIC]),
             rnd.choice([4 * nb, 8 * nb]), reqs, bs)


def test_rejections_and_exhausted_host_space(PK):
    a = PK.BlockAllocator(4)
    s = PK.Scheduler(a, 2, 64)
    with pytest.raises(PK.PkvError) as e:
        s.add_request(65, 1)
    assert e.value.status == PK.PKV_ERR_INVALID_ARG
    with pytest.raises(PK.PkvError) as e:
        s.add_request(40, 40)
    assert e.value.status == PK.PKV_ERR_OUT_OF_BLOCKS
    with pytest.raises(PK.PkvError):
        PK.Scheduler(a, 0, 64)
    # no host space: two requests that outgrow a 4-block pool together dead-lock
    # at the third step (request 0 needs a block, request 1 cannot leave)
    a2 = PK.BlockAllocator(4)
    s2 = PK.Scheduler(a2, 2, 64, PK.PKV_SCHED_CONTINUOUS, 0)
    m = SC.SchedulerModel(O.BlockAllocatorModel(4), 2, 64, SC.CONTINUOUS, 0)
    for sched in (s2, m):
        sched.add_request(31, 30)
        sched.add_request(31, 30)
    for _ in range(2):
        x, y = s2.step(), m.step()
        assert list(x.decode) == y.decode and list(x.prefill) == y.prefill
    with pytest.raises(PK.PkvError) as e:
        s2.step()
    assert e.value.status == PK.PKV_ERR_OUT_OF_BLOCKS
    with pytest.raises(RuntimeError):
        m.step()
