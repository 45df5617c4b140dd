"""The oracle at block sizes 8 and 32, pinned by what the paging must not
change: a fresh sequence takes ceil(n / P) blocks with slots
table[t // P] * P + t % P; gathering through the table returns exactly the rows
written; and the same logical rows placed with 8-, 16- or 32-token blocks (and
any shuffled pool) give bit-identical attention."""
import numpy as np
import pytest

import pkv_workloads as W
from oracle import pkv_oracle as O


@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("n", [1, 7, 8, 9, 31, 32, 33, 100])
def test_fresh_sequence_blocks_and_slots(bs, n):
    a = O.BlockAllocatorModel(40, bs, list(range(39, -1, -1)))
    s = a.create()
    slots, pairs = a.append_slots(s, n)
    t = a.block_table(s)
    assert len(t) == -(-n // bs) and not pairs
    assert slots == [t[i // bs] * bs + i % bs for i in range(n)]
    assert t == list(range(39, 39 - len(t), -1))        # first in first out from the given order


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attention_is_the_same_for_every_block_size(dtype):
    ctx = [1, 9, 16, 33, 70, 129]
    w = W._plain_decode("bs", 77, ctx, 4, 2, 64, dtype, pool_factor=1.7)
    outs = []
    for bs in (8, 16, 32):
        nb = sum(-(-c // bs) for c in ctx) + 5
        order = np.random.default_rng(bs).permutation(nb)
        r = O.replay(w.ops, w.k_rows, w.v_rows, nb, w.num_kv_heads, w.head_dim, order, block_size=bs)
        for s, c in zip(w.decode_seqs, ctx):
            got = O.gather_context(r.k_pool, r.alloc.block_table(s), c, bs)
            first = sum(ctx[:s])
            assert np.array_equal(got, w.k_rows[first:first + c])
        outs.append(O.decode_attention(w.q, r.k_pool, r.v_pool, [r.alloc.block_table(s) for s in w.decode_seqs],
                                       ctx, w.scale, block_size=bs))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])
