"""Decode and prefill at the edges of their sizes, against the oracle: more
sequences than the plan kernel's 1024 threads (three chunks of its scans),
empty contexts among them; a vector-ALU context of 70,000 tokens (69 partitions
of 1024, merged in nine chunks of eight) and a grouped-query context of 140,000
tokens on the matrix-core kernels, bf16 and float32 (137 partitions of 1024 for a
batch of three sequences); a 3000-query prefill chunk ending a 20,000-token context (hundreds of key tiles per wave, dozens of
row tiles), bf16 and float32, checked on its first, middle and last queries."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_kv_cache_171_amd as PK  # noqa: E402
import pkv_workloads as W  # noqa: E402
from oracle import pkv_oracle as O  # noqa: E402
from pkv_gpu_driver import GpuReplay  # noqa: E402

TOL = {"f32": 1e-5, "bf16": 2e-3}


def _check(w, sample=None):
    g = GpuReplay(w)
    r = O.replay(w.ops, w.k_rows, w.v_rows, w.num_blocks, w.num_kv_heads, w.head_dim, w.initial_free_order)
    out, tables, lens = g.decode()
    idx = list(range(len(w.decode_seqs))) if sample is None else sample
    ref = O.decode_attention(w.q[idx], r.k_pool, r.v_pool, [r.alloc.block_table(w.decode_seqs[i]) for i in idx],
                             [r.alloc.num_tokens(w.decode_seqs[i]) for i in idx], w.scale)
    err = float(np.abs(out[idx] - ref).max())
    assert err <= TOL[w.dtype], err
    return out, lens


def test_three_thousand_sequences_with_empty_contexts():
    print("case: max sizes, 3000 sequences", flush=True)
    rng = np.random.default_rng(81)
    ctx = rng.integers(0, 151, size=3000)
    ctx[::97] = 0
    w = W.from_lengths(81, ctx, 4, 4, 64, "f32")
    out, lens = _check(w)
    assert (np.asarray(lens) == 0).sum() >= 30
    assert np.all(out[np.asarray(lens) == 0] == 0)


def test_seventy_thousand_token_context_on_the_vector_kernel():
    print("case: max sizes, 70000-token MHA context", flush=True)
    w = W.from_lengths(82, [70000, 5, 1024, 1025], 2, 2, 128, "bf16")
    _check(w)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_hundred_forty_thousand_token_context_on_the_matrix_kernel(dtype):
    print(f"case: max sizes, 140000-token GQA context {dtype}", flush=True)
    w = W.from_lengths(83, [140000, 4097, 1], 8, 1, 128, dtype)
    _check(w)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_three_thousand_query_chunk_on_a_twenty_thousand_token_context(dtype):
    print(f"case: max sizes, prefill {dtype} 3000 queries at 20000", flush=True)
    ctx, n = 20000, 3000
    w = W.random_prefill(84, [ctx], [n], 8, 2, 128, dtype=dtype)
    g = GpuReplay(w)
    r = O.replay(w.ops, w.k_rows, w.v_rows, w.num_blocks, w.num_kv_heads, w.head_dim, w.initial_free_order)
    out, _, _ = g.prefill()
    assert np.isfinite(out).all()
    table = r.alloc.block_table(w.chunk_seqs[0])
    assert r.alloc.num_tokens(w.chunk_seqs[0]) == ctx
    one = np.array([0, 1], dtype=np.int32)
    err = 0.0
    # a query at chunk index i sits at position ctx - n + i: alone, it is the
    # one-query chunk of the context cut after it
    for i in (0, 1, 15, 16, 17, 1499, 1500):
        ref = O.prefill_chunk_attention(w.chunk_q[i:i + 1], one, r.k_pool, r.v_pool, [table], [ctx - n + i + 1],
                                        w.scale)
        err = max(err, float(np.abs(out[i:i + 1] - ref).max()))
    # the last 40 queries are the last 40 tokens of the whole context
    ref = O.prefill_chunk_attention(w.chunk_q[n - 40:], np.array([0, 40], dtype=np.int32), r.k_pool, r.v_pool,
                                    [table], [ctx], w.scale)
    err = max(err, float(np.abs(out[n - 40:] - ref).max()))
    assert err <= TOL[dtype], err
