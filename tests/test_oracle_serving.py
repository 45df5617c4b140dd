"""The oracle's continuous-batching loop on real rows, pinned by brute force:
every prefill and decode output it produces equals plain softmax attention of
that query over the request's own rows 0..position, taken straight from the
workload with no pool, table, slot or swap in between.  A dropped or misplaced
token anywhere (a wrong slot, a swap copy to the wrong block, a stale block)
changes some output."""
import math

import numpy as np
import pytest

import pkv_workloads as W
from oracle import pkv_oracle as O
from oracle import scheduler as SC
from oracle import serving as SV


def f64(bits):
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def direct(w, rid, pos):
    """softmax(scale q.k) v over positions 0..pos of request rid, per head."""
    a = int(w.row_start[rid])
    q = f64(w.q_rows[a + pos])
    K = f64(w.k_rows[a:a + pos + 1])
    V = f64(w.v_rows[a:a + pos + 1])
    G = w.num_heads // w.num_kv_heads
    out = np.empty((w.num_heads, w.head_dim))
    for h in range(w.num_heads):
        z = float(w.scale) * (K[:, h // G, :] @ q[h])
        e = np.exp(z - z.max())
        out[h] = (e @ V[:, h // G, :]) / e.sum()
    return out


@pytest.mark.parametrize("policy", [SC.CONTINUOUS, SC.STATIC])
def test_every_output_equals_attention_over_the_request_own_rows(policy):
    w = W.serving(seed=11, num_requests=10, hq=4, hkv=2, d=64, prompt_median=20, output_median=20,
                  max_prompt=60, max_output=50, num_blocks=12, max_num_seqs=4, max_num_batched_tokens=96,
                  num_host_blocks=48)
    m = SV.ServingModel(w, policy)
    swaps = 0
    produced = [0] * len(w.prompts)
    while True:
        x = m.step()
        st = x.step
        if not st.prefill and not st.decode:
            break
        swaps += len(st.swapped_out)
        row = 0
        for rid, n in zip(st.prefill, st.prefill_lens):
            for p in range(n):
                np.testing.assert_allclose(x.prefill_out[row], direct(w, rid, p), rtol=0, atol=1e-12)
                row += 1
            produced[rid] += 1
        for i, (rid, pos) in enumerate(zip(st.decode, x.decode_positions)):
            assert pos == w.prompts[rid] + produced[rid] - 1
            np.testing.assert_allclose(x.decode_out[i], direct(w, rid, pos), rtol=0, atol=1e-12)
            produced[rid] += 1
    assert produced == list(w.outputs)
    if policy == SC.CONTINUOUS:
        assert swaps > 0          # the pool is small enough that swapping happens


def test_swap_blocks_moves_whole_blocks_bit_for_bit():
    rng = np.random.default_rng(0)
    dev_k = rng.integers(0, 1 << 16, size=(6, 2, 16, 8), dtype=np.uint16)
    dev_v = rng.integers(0, 1 << 16, size=(6, 2, 16, 8), dtype=np.uint16)
    host_k = np.zeros((9, 2, 16, 8), dtype=np.uint16)
    host_v = np.zeros_like(host_k)
    k0, v0 = dev_k.copy(), dev_v.copy()
    O.swap_blocks(host_k, host_v, dev_k, dev_v, [(4, 0), (1, 7), (5, 3)])
    assert (host_k[[0, 7, 3]] == k0[[4, 1, 5]]).all() and (host_v[[0, 7, 3]] == v0[[4, 1, 5]]).all()
    assert (host_k[[1, 2, 4, 5, 6, 8]] == 0).all()
    dev_k[:] = 0
    dev_v[:] = 0
    O.swap_blocks(dev_k, dev_v, host_k, host_v, [(0, 2), (7, 0), (3, 5)])
    assert (dev_k[[2, 0, 5]] == k0[[4, 1, 5]]).all() and (dev_v[[2, 0, 5]] == v0[[4, 1, 5]]).all()
    assert (dev_k[[1, 3, 4]] == 0).all()
    f = np.full((3, 1, 16, 4), np.nan, dtype=np.float32)
    g = np.zeros_like(f)
    O.swap_blocks(g, g.copy(), f, f, [(2, 1)])
    assert np.isnan(g[1]).all() and not np.isnan(g[[0, 2]]).any()     # bits, not values
    with pytest.raises(ValueError):
        O.swap_blocks(host_k, host_v, dev_k, dev_v, [(0, 1), (2, 1)])


def test_serving_workload_fits_its_pool():
    w = W.serving()
    assert (w.prompts >= 1).all() and (w.outputs >= 1).all()
    assert (np.ceil((w.prompts + w.outputs) / 16) <= w.num_blocks).all()
    assert w.row_start[-1] == w.k_rows.shape[0] == w.q_rows.shape[0]
    assert w.scale == np.float32(1 / math.sqrt(w.head_dim))
