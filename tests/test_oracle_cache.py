"""Pins of the oracle's pool write and block copy (bit-exact byte moves)."""
import numpy as np
import pytest

from oracle import pkv_oracle as O
from pkv_workloads import f32_to_bf16_bits, parallel_sampling

P = 16


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_write_then_gather_returns_the_rows_and_touches_nothing_else(dtype):
    rng = np.random.default_rng(0)
    nb, hkv, d = 12, 3, 8
    base = rng.standard_normal((nb, hkv, P, d), dtype=np.float32)
    rows_k = rng.standard_normal((20, hkv, d), dtype=np.float32)
    rows_v = rng.standard_normal((20, hkv, d), dtype=np.float32)
    if dtype == "bf16":
        base, rows_k, rows_v = f32_to_bf16_bits(base), f32_to_bf16_bits(rows_k), f32_to_bf16_bits(rows_v)
    k, v = base.copy(), base.copy()
    table = [7, 2]
    slots = [table[t // P] * P + t % P for t in range(20)]
    slots_with_skip = list(slots)
    slots_with_skip[5] = -1
    O.write_cache(k, v, rows_k, rows_v, slots_with_skip)
    got = O.gather_context(k, table, 20)
    for t in range(20):
        if t == 5:
            assert np.array_equal(got[t].view(np.uint8), base[7, :, 5].view(np.uint8))
        else:
            assert np.array_equal(got[t].view(np.uint8), rows_k[t].view(np.uint8))
    assert np.array_equal(O.gather_context(v, table, 20)[6], rows_v[6])
    untouched = [b for b in range(nb) if b not in table]
    assert np.array_equal(k[untouched].view(np.uint8), base[untouched].view(np.uint8))
    assert np.array_equal(k[2, :, 4:].view(np.uint8), base[2, :, 4:].view(np.uint8))


def test_write_preserves_nan_payload_bits():
    k = np.zeros((2, 1, P, 4), np.float32)
    v = np.zeros_like(k)
    row = np.array([[[np.nan, -0.0, np.inf, 1.5]]], np.float32)
    row.view(np.uint32)[0, 0, 0] = 0x7FC0DEAD
    O.write_cache(k, v, row, row, [17])
    assert k.view(np.uint32)[1, 0, 1, 0] == 0x7FC0DEAD
    assert k.view(np.uint32)[1, 0, 1, 1] == 0x80000000


def test_duplicate_slot_in_one_call_is_rejected():
    k = np.zeros((2, 1, P, 4), np.float32)
    with pytest.raises(ValueError):
        O.write_cache(k, k.copy(), np.zeros((2, 1, 4), np.float32), np.zeros((2, 1, 4), np.float32), [3, 3])


def test_copy_blocks_reads_the_pool_before_the_call():
    rng = np.random.default_rng(1)
    k = f32_to_bf16_bits(rng.standard_normal((6, 2, P, 8), dtype=np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((6, 2, P, 8), dtype=np.float32))
    k0, v0 = k.copy(), v.copy()
    O.copy_blocks(k, v, [(1, 4), (1, 5), (2, 0)])
    assert np.array_equal(k[4], k0[1]) and np.array_equal(k[5], k0[1]) and np.array_equal(k[0], k0[2])
    assert np.array_equal(v[4], v0[1]) and np.array_equal(v[0], v0[2])
    for b in (1, 2, 3):
        assert np.array_equal(k[b], k0[b]) and np.array_equal(v[b], v0[b])
    with pytest.raises(ValueError):
        O.copy_blocks(k, v, [(1, 4), (2, 4)])
    with pytest.raises(ValueError):
        O.copy_blocks(k, v, [(1, 4), (4, 3)])


def test_forked_samples_equal_unshared_copies():
    """Sharing prompt blocks through fork + copy-on-write gives the same pool
    contents per sequence, and the same attention, as writing every sample's
    prompt separately."""
    w = parallel_sampling(seed=11, groups=2, samples=4, prompt=40, tail_hi=40, hq=2, d=16)
    shared = O.replay(w.ops, w.k_rows, w.v_rows, w.num_blocks, w.num_kv_heads, w.head_dim,
                      w.initial_free_order)
    # unshared script: every sample writes its prompt rows again, then its tail
    parent = {}
    rows_of = {}
    r, n_seq = 0, 0
    for op in w.ops:
        if op[0] == "create":
            parent[n_seq] = None; n_seq += 1
        elif op[0] == "fork":
            parent[n_seq] = op[1]; n_seq += 1
        elif op[0] == "append":
            rows_of.setdefault(op[1], []).append((r, r + op[2]))
            r += op[2]
    ops, rows_k, rows_v = [], [], []
    for s in range(n_seq):
        spans = ([] if parent[s] is None else rows_of[parent[s]][:1]) + rows_of[s]
        idx = np.concatenate([np.arange(a, b) for a, b in spans])
        ops += [("create",), ("append", s, len(idx)), ("flush",)]
        rows_k.append(w.k_rows[idx])
        rows_v.append(w.v_rows[idx])
    alone = O.replay(ops, np.concatenate(rows_k), np.concatenate(rows_v), 200, w.num_kv_heads,
                     w.head_dim)
    for s in w.decode_seqs:
        n = shared.alloc.num_tokens(s)
        assert n == alone.alloc.num_tokens(s)
        assert np.array_equal(O.gather_context(shared.k_pool, shared.alloc.block_table(s), n),
                              O.gather_context(alone.k_pool, alone.alloc.block_table(s), n))
    t_sh = [shared.alloc.block_table(s) for s in w.decode_seqs]
    t_al = [alone.alloc.block_table(s) for s in w.decode_seqs]
    lens = [shared.alloc.num_tokens(s) for s in w.decode_seqs]
    o1 = O.decode_attention(w.q, shared.k_pool, shared.v_pool, t_sh, lens, w.scale)
    o2 = O.decode_attention(w.q, alone.k_pool, alone.v_pool, t_al, lens, w.scale)
    assert np.array_equal(o1, o2)
