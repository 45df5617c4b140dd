"""Plant plausible mistakes in the oracle (on the CPU) and check a pin catches each.

Every mutant replaces one oracle function by a copy with a single slip -- a
dropped scale, a flipped sign, a wrong head or slot index, an off-by-one causal
position, a wrong merge factor, a different free-list or copy-on-write rule --
and at least one pin test must then fail.
"""
import collections
import math

import numpy as np
import pytest

from oracle import pkv_oracle as O
import test_oracle_allocator as TA
import test_oracle_attention as TT
import test_oracle_cache as TC

P = 16


def _fails(*checks):
    for c in checks:
        try:
            c()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


ATTN_PINS = [
    TT.test_ctx1_returns_the_single_value_row_exactly,
    TT.test_zero_query_gives_mean_of_values,
    TT.test_two_tokens_follow_the_logistic_weight_and_use_the_scale,
    TT.test_dominant_key_selects_its_value,
    lambda: TT.test_contiguous_placement_matches_torch_sdpa(8, 2, "f32"),
    lambda: TT.test_contiguous_placement_matches_torch_sdpa(4, 4, "f32"),
    TT.test_physical_block_relabelling_leaves_outputs_bit_identical,
    TT.test_nan_in_unused_slots_never_reaches_the_output,
    TT.test_chunk_queries_match_sdpa_with_bottom_right_causal_mask_and_decode,
    TT.test_split_context_merge_equals_unsplit_softmax,
]


def _softmax_no_scale(qv, keys, values, scale):
    z = keys @ qv
    w = np.exp(z - z.max())
    return (w @ values) / w.sum()


def _softmax_flipped(qv, keys, values, scale):
    z = scale * (keys @ qv)
    w = np.exp(z.min() - z)
    return (w @ values) / w.sum()


def _gather_offset_slip(pool, table, ctx, block_size=P):
    t = np.arange(ctx)
    blocks = np.asarray(table, dtype=np.int64)[t // block_size]
    return pool[blocks, :, (t + 1) % block_size, :]


def _gather_swapped(pool, table, ctx, block_size=P):
    t = np.arange(ctx)
    idx = np.asarray(table, dtype=np.int64)
    return pool[idx[np.minimum(t % block_size, len(idx) - 1)], :, t // block_size % block_size, :]


def _merge_wrong_sign(ms, ls, accs):
    M = max(ms)
    num = sum(acc * math.exp(M - m) for m, acc in zip(ms, accs))
    den = sum(l * math.exp(M - m) for m, l in zip(ms, ls))
    return num / den


@pytest.mark.parametrize("name,target,mutant", [
    ("dropped scale", "softmax_attention", _softmax_no_scale),
    ("flipped exponent", "softmax_attention", _softmax_flipped),
    ("slot offset off by one", "gather_context", _gather_offset_slip),
    ("block / offset swapped", "gather_context", _gather_swapped),
    ("kv head h % Hkv", "kv_head_of", lambda h, hq, hkv: h % hkv),
    ("merge factor inverted", "merge_partials", _merge_wrong_sign),
])
def test_attention_mutants_are_caught(monkeypatch, name, target, mutant):
    monkeypatch.setattr(O, target, mutant)
    assert _fails(*ATTN_PINS), name


def test_causal_position_off_by_one_is_caught(monkeypatch):
    real = O.softmax_attention

    def chunk(q, qsl, k_pool, v_pool, tables, lens, scale, block_size=P):
        # same as the oracle but each query sees one key fewer
        Tq, Hq, d = q.shape
        Hkv = k_pool.shape[1]
        out = np.zeros((Tq, Hq, d))
        for s in range(len(qsl) - 1):
            a, b = int(qsl[s]), int(qsl[s + 1])
            ctx, n = int(lens[s]), b - a
            K = O.storage_to_f64(O.gather_context(k_pool, tables[s], ctx))
            V = O.storage_to_f64(O.gather_context(v_pool, tables[s], ctx))
            for i in range(n):
                p = max(0, ctx - n + i - 1)
                qi = O.storage_to_f64(q[a + i])
                for h in range(Hq):
                    g = O.kv_head_of(h, Hq, Hkv)
                    out[a + i, h] = real(qi[h], K[:p + 1, g], V[:p + 1, g], float(np.float32(scale)))
        return out

    monkeypatch.setattr(O, "prefill_chunk_attention", chunk)
    assert _fails(TT.test_chunk_queries_match_sdpa_with_bottom_right_causal_mask_and_decode)


ALLOC_PINS = [
    TA.test_blocks_come_first_in_first_out_and_return_to_the_back,
    TA.test_fork_shares_every_block_and_partial_shared_block_is_copied_once_per_writer,
    TA.test_full_shared_last_block_is_not_copied,
    TA.test_out_of_blocks_changes_nothing,
    TA.test_parallel_sampling_block_counts_match_the_closed_form,
    lambda: TA.test_fresh_sequence_gets_ceil_blocks_and_consecutive_slots(33),
    TC.test_forked_samples_equal_unshared_copies,
]


class _LifoModel(O.BlockAllocatorModel):
    def free_seq(self, sid):
        for b in self.tables[sid]:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.appendleft(b)
        del self.tables[sid], self.lens[sid]


class _CopyFullToo(O.BlockAllocatorModel):
    def append_slots(self, sid, n):
        table = self.tables[sid]
        if n and table and self.lens[sid] % self.block_size == 0 and self.ref[table[-1]] > 1:
            old = table[-1]
            b = self.free.popleft()
            self.ref[old] -= 1
            self.ref[b] = 1
            table[-1] = b
            slots, pairs = super().append_slots(sid, n)
            return slots, [(old, b)] + pairs
        return super().append_slots(sid, n)


class _NeverCopy(O.BlockAllocatorModel):
    def append_slots(self, sid, n):
        ref = self.ref
        self.ref = collections.defaultdict(int)  # every block looks unshared
        try:
            return super().append_slots(sid, n)
        finally:
            for b, r in self.ref.items():
                ref[b] = r
            self.ref = ref


class _NotAtomic(O.BlockAllocatorModel):
    def blocks_needed(self, sid, n):
        return 0


@pytest.mark.parametrize("name,cls", [
    ("LIFO free list", _LifoModel),
    ("copies full shared blocks", _CopyFullToo),
    ("never copies on write", _NeverCopy),
    ("fails half-way on a short pool", _NotAtomic),
])
def test_allocator_mutants_are_caught(monkeypatch, name, cls):
    monkeypatch.setattr(O, "BlockAllocatorModel", cls)
    assert _fails(*ALLOC_PINS), name


def test_write_with_block_and_offset_swapped_is_caught(monkeypatch):
    def bad_write(k_pool, v_pool, k, v, slot_mapping, block_size=P):
        for t, slot in enumerate(slot_mapping):
            if slot < 0:
                continue
            off, blk = divmod(int(slot), block_size)
            k_pool[blk % k_pool.shape[0], :, off % block_size] = k[t]
            v_pool[blk % v_pool.shape[0], :, off % block_size] = v[t]

    monkeypatch.setattr(O, "write_cache", bad_write)
    assert _fails(lambda: TC.test_write_then_gather_returns_the_rows_and_touches_nothing_else("f32"),
                  TC.test_forked_samples_equal_unshared_copies)


def _widen_as_fp16(a):
    if a.dtype == np.uint16:
        return a.view(np.float16).astype(np.float64)
    return a.astype(np.float64)


def _widen_byte_swapped(a):
    if a.dtype == np.uint16:
        return (a.byteswap().astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _widen_truncated_to_f32_low_half(a):
    if a.dtype == np.uint16:
        return a.astype(np.uint32).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


@pytest.mark.parametrize("name,mutant", [
    ("bf16 bits read as fp16", _widen_as_fp16),
    ("bf16 bytes swapped", _widen_byte_swapped),
    ("bf16 bits in the low half of a float32", _widen_truncated_to_f32_low_half),
])
def test_storage_widening_mutants_are_caught(monkeypatch, name, mutant):
    import test_oracle_storage as TS
    monkeypatch.setattr(O, "storage_to_f64", mutant)
    assert _fails(TS.test_bf16_widening_matches_torch_bfloat16_on_every_bit_pattern,
                  TS.test_bf16_widening_of_fixed_patterns), name
