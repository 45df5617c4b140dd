"""Pins of the oracle's attention against things other than itself.

Closed forms (ctx = 1, q = 0, constant values, two-token logistic, a dominant
key), a library routine (torch's scaled_dot_product_attention in float64 on the
CPU, including its grouped-query convention and a bottom-right causal mask),
the block-permutation and NaN-poison invariances of paging, and the
log-sum-exp merge of split contexts.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import pkv_oracle as O
from pkv_workloads import f32_to_bf16_bits

P = 16


def _pool_with_context(rng, ctxs, hkv, d, dtype, nb=None, contiguous=False):
    """A pool holding ctxs[s] random tokens per sequence and their tables."""
    need = sum(-(-c // P) for c in ctxs)
    nb = nb or need + 3
    order = np.arange(nb) if contiguous else rng.permutation(nb)
    k = rng.standard_normal((nb, hkv, P, d), dtype=np.float32)
    v = rng.standard_normal((nb, hkv, P, d), dtype=np.float32)
    if dtype == "bf16":
        k, v = f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    tables, i = [], 0
    for c in ctxs:
        nblk = -(-c // P)
        tables.append([int(b) for b in order[i:i + nblk]])
        i += nblk
    return k, v, tables


def _q(rng, s, hq, d, dtype):
    q = rng.standard_normal((s, hq, d), dtype=np.float32)
    return f32_to_bf16_bits(q) if dtype == "bf16" else q


def test_ctx1_returns_the_single_value_row_exactly():
    rng = np.random.default_rng(0)
    k, v, tables = _pool_with_context(rng, [1, 1], 2, 64, "f32")
    q = _q(rng, 2, 4, 64, "f32")
    o = O.decode_attention(q, k, v, tables, [1, 1], 0.125)
    for s in range(2):
        for h in range(4):
            g = h // 2
            assert np.array_equal(o[s, h], v[tables[s][0], g, 0].astype(np.float64))


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(1)
    k, v, tables = _pool_with_context(rng, [37], 1, 64, "f32")
    q = np.zeros((1, 1, 64), np.float32)
    o = O.decode_attention(q, k, v, tables, [37], 0.125)
    rows = np.stack([v[tables[0][t // P], 0, t % P] for t in range(37)]).astype(np.float64)
    np.testing.assert_allclose(o[0, 0], rows.mean(axis=0), rtol=0, atol=1e-14)


def test_identical_keys_give_mean_of_values():
    # every key the same: every score the same, so the softmax is uniform
    # whatever the query
    rng = np.random.default_rng(11)
    k, v, tables = _pool_with_context(rng, [29], 2, 64, "f32")
    key = rng.standard_normal((2, 64)).astype(np.float32)
    for t in range(29):
        k[tables[0][t // P], :, t % P] = key
    q = _q(rng, 1, 4, 64, "f32")
    o = O.decode_attention(q, k, v, tables, [29], 0.125)
    for h in range(4):
        g = h // 2
        rows = np.stack([v[tables[0][t // P], g, t % P] for t in range(29)]).astype(np.float64)
        np.testing.assert_allclose(o[0, h], rows.mean(axis=0), rtol=0, atol=1e-14)


def test_constant_value_rows_give_that_row():
    rng = np.random.default_rng(2)
    k, v, tables = _pool_with_context(rng, [45], 1, 32, "f32")
    row = rng.standard_normal(32).astype(np.float32)
    v[:] = row
    q = _q(rng, 1, 1, 32, "f32")
    o = O.decode_attention(q, k, v, tables, [45], 0.3)
    np.testing.assert_allclose(o[0, 0], row.astype(np.float64), rtol=1e-14, atol=1e-15)


def test_two_tokens_follow_the_logistic_weight_and_use_the_scale():
    rng = np.random.default_rng(3)
    k, v, tables = _pool_with_context(rng, [2], 1, 16, "f32")
    q = _q(rng, 1, 1, 16, "f32")
    scale = np.float32(0.7)
    k0 = k[tables[0][0], 0, 0].astype(np.float64)
    k1 = k[tables[0][0], 0, 1].astype(np.float64)
    v0 = v[tables[0][0], 0, 0].astype(np.float64)
    v1 = v[tables[0][0], 0, 1].astype(np.float64)
    qd = q[0, 0].astype(np.float64)
    gap = float(scale) * (np.dot(qd, k0) - np.dot(qd, k1))
    w0 = scipy.special.expit(gap)
    expect = w0 * v0 + (1.0 - w0) * v1
    o = O.decode_attention(q, k, v, tables, [2], scale)
    np.testing.assert_allclose(o[0, 0], expect, rtol=1e-13, atol=1e-14)
    # doubling the scale must change the answer (the scale is not dropped)
    o2 = O.decode_attention(q, k, v, tables, [2], np.float32(1.4))
    assert not np.allclose(o2, o)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(4)
    k, v, tables = _pool_with_context(rng, [40], 1, 64, "f32")
    k *= np.float32(0.01)
    target = 23
    qv = rng.standard_normal(64).astype(np.float32)
    k[tables[0][target // P], 0, target % P] = qv * 4
    o = O.decode_attention(qv.reshape(1, 1, 64), k, v, tables, [40], 1.0)
    np.testing.assert_allclose(o[0, 0], v[tables[0][target // P], 0, target % P], atol=1e-9)


@pytest.mark.parametrize("hq,hkv,dtype", [(4, 4, "f32"), (8, 2, "f32"), (8, 8, "bf16"), (16, 2, "bf16")])
def test_contiguous_placement_matches_torch_sdpa(hq, hkv, dtype):
    rng = np.random.default_rng(5 + hq + hkv)
    d = 64
    ctxs = [1, 15, 16, 17, 70, 129]
    k, v, tables = _pool_with_context(rng, ctxs, hkv, d, dtype, contiguous=True)
    q = _q(rng, len(ctxs), hq, d, dtype)
    scale = np.float32(1 / math.sqrt(d))
    o = O.decode_attention(q, k, v, tables, ctxs, scale)
    qf, kf, vf = O.storage_to_f64(q), O.storage_to_f64(k), O.storage_to_f64(v)
    for s, c in enumerate(ctxs):
        # contiguous placement: tokens are the first c rows of the flattened blocks
        first = tables[s][0]
        kk = kf[first:first + len(tables[s])].transpose(1, 0, 2, 3).reshape(hkv, -1, d)[:, :c]
        vv = vf[first:first + len(tables[s])].transpose(1, 0, 2, 3).reshape(hkv, -1, d)[:, :c]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qf[s][:, None, :]), torch.from_numpy(np.ascontiguousarray(kk)),
            torch.from_numpy(np.ascontiguousarray(vv)), scale=float(scale),
            enable_gqa=(hq != hkv))
        np.testing.assert_allclose(o[s], ref[:, 0, :].numpy(), rtol=0, atol=1e-12)


def test_physical_block_relabelling_leaves_outputs_bit_identical():
    rng = np.random.default_rng(6)
    ctxs = [3, 16, 33, 80]
    k, v, tables = _pool_with_context(rng, ctxs, 2, 32, "bf16")
    q = _q(rng, 4, 4, 32, "bf16")
    o = O.decode_attention(q, k, v, tables, ctxs, 0.2)
    pi = rng.permutation(k.shape[0])
    k2, v2 = np.empty_like(k), np.empty_like(v)
    k2[pi], v2[pi] = k, v
    t2 = [[int(pi[b]) for b in t] for t in tables]
    o2 = O.decode_attention(q, k2, v2, t2, ctxs, 0.2)
    assert np.array_equal(o, o2)


def test_nan_in_unused_slots_never_reaches_the_output():
    rng = np.random.default_rng(7)
    ctxs = [5, 17, 32, 1]
    k, v, tables = _pool_with_context(rng, ctxs, 2, 32, "f32")
    q = _q(rng, 4, 2, 32, "f32")
    o = O.decode_attention(q, k, v, tables, ctxs, 0.25)
    live = np.zeros(k.shape[:1] + k.shape[2:3], dtype=bool)  # [NB, P]
    for t, c in zip(tables, ctxs):
        for i in range(c):
            live[t[i // P], i % P] = True
    kp, vp = k.copy(), v.copy()
    kp.transpose(0, 2, 1, 3)[~live] = np.nan
    vp.transpose(0, 2, 1, 3)[~live] = np.nan
    o2 = O.decode_attention(q, kp, vp, tables, ctxs, 0.25)
    assert np.isfinite(o2).all() and np.array_equal(o, o2)


def test_zero_context_gives_zero_row():
    rng = np.random.default_rng(8)
    k, v, tables = _pool_with_context(rng, [4], 1, 16, "f32")
    q = _q(rng, 2, 1, 16, "f32")
    o = O.decode_attention(q, k, v, [tables[0], []], [4, 0], 0.25)
    assert np.array_equal(o[1], np.zeros((1, 16)))


def test_split_context_merge_equals_unsplit_softmax():
    rng = np.random.default_rng(9)
    keys = rng.standard_normal((300, 64))
    vals = rng.standard_normal((300, 64))
    qv = rng.standard_normal(64) * 2
    full = O.softmax_attention(qv, keys, vals, 0.125)
    for cuts in ([300], [1, 299], [100, 100, 100], [7, 13, 80, 200]):
        bounds = np.cumsum([0] + cuts)
        parts = [O.attention_partial(qv, keys[a:b], vals[a:b], 0.125) for a, b in zip(bounds[:-1], bounds[1:])]
        o = O.merge_partials([p[0] for p in parts], [p[1] for p in parts], [p[2] for p in parts])
        np.testing.assert_allclose(o, full, rtol=0, atol=1e-13)
    # a single partition is acc / l
    m, l, acc = O.attention_partial(qv, keys, vals, 0.125)
    np.testing.assert_allclose(acc / l, full, atol=1e-14)


def test_chunk_queries_match_sdpa_with_bottom_right_causal_mask_and_decode():
    rng = np.random.default_rng(10)
    hq, hkv, d = 4, 2, 32
    ctxs = [40, 23]
    n_q = [9, 23]
    k, v, tables = _pool_with_context(rng, ctxs, hkv, d, "bf16", contiguous=True)
    qsl = np.array([0, n_q[0], n_q[0] + n_q[1]], dtype=np.int32)
    q = _q(rng, qsl[-1], hq, d, "bf16")
    scale = np.float32(0.17)
    o = O.prefill_chunk_attention(q, qsl, k, v, tables, ctxs, scale)
    qf, kf, vf = O.storage_to_f64(q), O.storage_to_f64(k), O.storage_to_f64(v)
    for s, c in enumerate(ctxs):
        first = tables[s][0]
        kk = kf[first:first + len(tables[s])].transpose(1, 0, 2, 3).reshape(hkv, -1, d)[:, :c]
        vv = vf[first:first + len(tables[s])].transpose(1, 0, 2, 3).reshape(hkv, -1, d)[:, :c]
        qq = qf[qsl[s]:qsl[s + 1]].transpose(1, 0, 2)
        mask = torch.ones(n_q[s], c, dtype=torch.bool).tril(diagonal=c - n_q[s])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(np.ascontiguousarray(qq)), torch.from_numpy(np.ascontiguousarray(kk)),
            torch.from_numpy(np.ascontiguousarray(vv)), attn_mask=mask, scale=float(scale),
            enable_gqa=True)
        np.testing.assert_allclose(o[qsl[s]:qsl[s + 1]], ref.numpy().transpose(1, 0, 2), atol=1e-12)
        # each chunk query equals a decode query over the prefix that ends at its
        # position (the chunk form sums in another order: equal to rounding)
        for i in range(n_q[s]):
            p = c - n_q[s] + i
            od = O.decode_attention(q[qsl[s] + i][None], k, v, [tables[s]], [p + 1], scale)
            np.testing.assert_allclose(od[0], o[qsl[s] + i], rtol=0, atol=1e-13)
