"""Seeded synthetic inputs for the paged KV-cache decode path.

This module only *draws inputs*: context lengths, a physical-block permutation,
query and key/value rows, and a script of allocator operations (create / fork /
append) that a caller replays on its own allocator.  It holds none of the
method's arithmetic -- no slot or block-table computation, no cache write, no
attention -- so that the HIP path and the CPU oracle can both consume the same
inputs while sharing no code.

Shapes and distributions follow the five workloads of the paged decode study:

1. ``tiny``  -- 4 sequences with context lengths [5, 50, 8, 12] (the first four
   request lengths of the slot-simulation example in the Ultralytics glossary
   page "Continuous Batching", section on iteration-level scheduling), 4 MHA
   heads, head_dim 64, fp32, 64 physical blocks in a seeded random order.
2. ``13b``   -- 64 sequences, 40 MHA heads, head_dim 128, bf16, context lengths
   lognormal (median 200, sigma 1.0) clipped to [1, 2048] -- the right-skewed
   length mix with mean 200 / max 2048 used in "Batching Continuo y
   PagedAttention" (cruxr.ai), section "Por qué el batching estático
   desperdicia GPUs"; pool = ceil(1.2 x blocks needed), shuffled.
3. ``gqa``   -- 256 sequences, 64 query / 8 KV heads, head_dim 128, bf16,
   context lengths uniform in [128, 4096], pool 1.2x, shuffled.
4. ``fork``  -- 32 groups x 8 parallel samples sharing a 1000-token prompt
   (62 full blocks + 1 partial block), per-sample generated tails uniform in
   [1, 512], 40 MHA heads, head_dim 128, bf16, pool 1.2x, shuffled.
5. ``long``  -- 16 decode sequences at context 32768 plus 4 prefill chunks of
   512 causal queries that end 8192-token contexts, 32 query / 8 KV heads,
   head_dim 128, bf16, pool sized exactly, shuffled.

All values are drawn with ``numpy.random.default_rng(seed)`` (seed = workload
number unless given).  Normal draws are float32 N(0, 1); for bf16 workloads
they are rounded to bf16 with round-to-nearest-even and carried as raw uint16
bits, so every consumer sees identical bits.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Tuple

import numpy as np

BLOCK_SIZE = 16

# Operation script entries (replayed in order by the consumer):
#   ("create",)              -> new sequence; ids are assigned 0, 1, 2, ... in op order
#   ("fork", parent_id)      -> new sequence sharing the parent's blocks
#   ("append", seq_id, n)    -> n new tokens for seq_id; their K/V rows are the next
#                               n rows of Workload.k_rows / v_rows
#   ("flush",)               -> apply pending block copies, then pending row writes
Op = Tuple


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even), returned as uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bits (uint16) to float32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str                    # "f32" or "bf16": storage dtype of q, K and V
    num_heads: int                # query heads Hq
    num_kv_heads: int             # KV heads Hkv
    head_dim: int
    num_blocks: int               # physical pool size NB
    initial_free_order: np.ndarray  # int32 [NB], a permutation of range(NB)
    ops: List[Op]                 # allocator script
    k_rows: np.ndarray            # [T_total, Hkv, d] storage values (float32 or uint16 bits)
    v_rows: np.ndarray
    decode_seqs: List[int]        # sequence ids that carry one decode query each
    q: np.ndarray                 # [len(decode_seqs), Hq, d] storage values
    scale: np.float32             # softmax scale 1/sqrt(d), rounded to fp32
    # chunked-prefill queries (workload 5 only)
    chunk_seqs: List[int] = dataclasses.field(default_factory=list)
    chunk_q: Optional[np.ndarray] = None          # [Tq, Hq, d]
    chunk_query_start_loc: Optional[np.ndarray] = None  # int32 [len(chunk_seqs)+1]
    block_size: int = BLOCK_SIZE

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return x if dtype == "f32" else f32_to_bf16_bits(x)


def _rows(rng, n_tokens: int, hkv: int, d: int, dtype: str, chunk_tokens: int = 1 << 16) -> np.ndarray:
    out = np.empty((n_tokens, hkv, d), dtype=np.float32 if dtype == "f32" else np.uint16)
    for t0 in range(0, n_tokens, chunk_tokens):
        t1 = min(n_tokens, t0 + chunk_tokens)
        out[t0:t1] = _normal(rng, (t1 - t0, hkv, d), dtype)
    return out


def lognormal_lengths(rng, n: int, median: float = 200.0, sigma: float = 1.0,
                      lo: int = 1, hi: int = 2048) -> np.ndarray:
    """clip(rint(exp(N(ln median, sigma))), lo, hi) as int32 (rint = half-to-even)."""
    x = np.exp(rng.normal(math.log(median), sigma, size=n))
    return np.clip(np.rint(x), lo, hi).astype(np.int32)


def _blocks_for(n_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    # pool sizing only: number of pages that n tokens occupy
    return -(-int(n_tokens) // block_size)


def _plain_decode(name, seed, ctx, hq, hkv, d, dtype, num_blocks=None, pool_factor=1.2,
                  with_rows=True, block_size=BLOCK_SIZE) -> Workload:
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx, dtype=np.int32)
    need = sum(_blocks_for(c, block_size) for c in ctx)
    nb = int(num_blocks) if num_blocks is not None else int(math.ceil(pool_factor * need))
    perm = rng.permutation(nb).astype(np.int32)
    q = _normal(rng, (len(ctx), hq, d), dtype)
    total = int(ctx.sum())
    if with_rows:
        k_rows = _rows(rng, total, hkv, d, dtype)
        v_rows = _rows(rng, total, hkv, d, dtype)
    else:
        k_rows = v_rows = np.empty((0, hkv, d), dtype=np.float32 if dtype == "f32" else np.uint16)
    ops: List[Op] = []
    for s, c in enumerate(ctx):
        ops.append(("create",))
        ops.append(("append", s, int(c)))
    ops.append(("flush",))
    scale = np.float32(1.0 / math.sqrt(d))
    return Workload(name, dtype, hq, hkv, d, nb, perm, ops, k_rows, v_rows,
                    list(range(len(ctx))), q, scale, block_size=block_size)


def tiny(seed: int = 1) -> Workload:
    """Workload 1: 4 sequences, ctx [5, 50, 8, 12], 4 MHA heads, d 64, fp32, 64 blocks."""
    return _plain_decode("tiny", seed, [5, 50, 8, 12], 4, 4, 64, "f32", num_blocks=64)


def shaped_13b_lengths(seed: int = 2, num_seqs: int = 64) -> np.ndarray:
    return lognormal_lengths(np.random.default_rng(seed), num_seqs)


def shaped_13b(seed: int = 2, num_seqs: int = 64, with_rows: bool = True, block_size: int = BLOCK_SIZE) -> Workload:
    """Workload 2: 64 seqs, 40 MHA heads, d 128, bf16, lognormal lengths, pool 1.2x
    (of the pages needed at ``block_size``)."""
    rng = np.random.default_rng(seed)
    ctx = lognormal_lengths(rng, num_seqs)
    return _plain_decode("13b", seed + 1000, ctx, 40, 40, 128, "bf16", with_rows=with_rows, block_size=block_size)


def gqa(seed: int = 3, num_seqs: int = 256, lo: int = 128, hi: int = 4096,
        with_rows: bool = True, block_size: int = BLOCK_SIZE) -> Workload:
    """Workload 3: 256 seqs, 64 q / 8 KV heads, d 128, bf16, ctx U[128, 4096], pool 1.2x
    (of the pages needed at ``block_size``)."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(lo, hi + 1, size=num_seqs).astype(np.int32)
    return _plain_decode("gqa", seed + 1000, ctx, 64, 8, 128, "bf16", with_rows=with_rows, block_size=block_size)


def parallel_sampling(seed: int = 4, groups: int = 32, samples=8, prompt=1000,
                      tail_lo: int = 1, tail_hi: int = 512, hq: int = 40, d: int = 128,
                      with_rows: bool = True, hkv: Optional[int] = None,
                      block_size: int = BLOCK_SIZE, dtype: str = "bf16") -> Workload:
    """Workload 4: groups x samples forks of one prompt each; tails U[1, 512].

    Script per group: create the prompt sequence (it is sample 0), append the
    prompt, flush, fork it samples-1 times, then append each sample's tail in
    sample order (a tail of 0 appends nothing), flush.  Every sample carries
    one decode query; the samples of a group are consecutive in decode_seqs.
    For parity cases ``samples`` and ``prompt`` may also be per-group lists,
    ``hkv`` < hq gives grouped-query heads and ``dtype`` "f32" float32 pools
    (the same draws, not rounded to bf16).
    """
    rng = np.random.default_rng(seed)
    hkv = hq if hkv is None else hkv
    n_samples = [int(x) for x in (samples if np.ndim(samples) else [samples] * groups)]
    prompts = [int(x) for x in (prompt if np.ndim(prompt) else [prompt] * groups)]
    tails = [rng.integers(tail_lo, tail_hi + 1, size=n).astype(np.int32) for n in n_samples]
    # pool sizing (an upper bound on the blocks in use, times 1.2): the prompt's
    # pages once per group, plus per sample one page of headroom and the tail's pages
    need = sum(_blocks_for(p, block_size) for p in prompts) + \
        sum(_blocks_for(int(t), block_size) + 1 for ts in tails for t in ts)
    nb = int(math.ceil(1.2 * need))
    perm = rng.permutation(nb).astype(np.int32)
    ops: List[Op] = []
    decode_seqs: List[int] = []
    next_id = 0
    for g in range(groups):
        root = next_id
        ops.append(("create",)); next_id += 1
        ops.append(("append", root, prompts[g]))
        ops.append(("flush",))
        members = [root]
        for _ in range(n_samples[g] - 1):
            ops.append(("fork", root)); members.append(next_id); next_id += 1
        for i, s in enumerate(members):
            if tails[g][i] > 0:
                ops.append(("append", s, int(tails[g][i])))
        ops.append(("flush",))
        decode_seqs.extend(members)
    total = sum(prompts) + int(sum(int(ts.sum()) for ts in tails))
    q = _normal(rng, (len(decode_seqs), hq, d), dtype)
    if with_rows:
        k_rows = _rows(rng, total, hkv, d, dtype)
        v_rows = _rows(rng, total, hkv, d, dtype)
    else:
        k_rows = v_rows = np.empty((0, hkv, d), dtype=np.float32 if dtype == "f32" else np.uint16)
    w = Workload("fork", dtype, hq, hkv, d, nb, perm, ops, k_rows, v_rows, decode_seqs, q,
                 np.float32(1.0 / math.sqrt(d)), block_size=block_size)
    w.tails = np.array(tails) if len(set(n_samples)) == 1 else tails  # type: ignore[attr-defined]
    w.prompt = prompt  # type: ignore[attr-defined]
    w.group_start = np.concatenate([[0], np.cumsum(n_samples)]).astype(np.int32)  # type: ignore[attr-defined]
    return w


def long_mix(seed: int = 5, n_decode: int = 16, decode_ctx: int = 32768, n_chunks: int = 4,
             chunk: int = 512, chunk_ctx: int = 8192, hq: int = 32, hkv: int = 8, d: int = 128,
             with_rows: bool = True) -> Workload:
    """Workload 5: 16 decode seqs at 32768 + 4 causal chunks of 512 ending 8192-token contexts.

    Sequences 0..n_decode-1 are decode sequences; the chunk sequences follow.
    A chunk sequence's last ``chunk`` tokens are the chunk's own tokens; their
    K/V rows are appended in the same script as the cached prefix.
    """
    rng = np.random.default_rng(seed)
    need = n_decode * _blocks_for(decode_ctx) + n_chunks * _blocks_for(chunk_ctx)
    perm = rng.permutation(need).astype(np.int32)
    ops: List[Op] = []
    for s in range(n_decode):
        ops.append(("create",)); ops.append(("append", s, decode_ctx))
    chunk_seqs = []
    for c in range(n_chunks):
        s = n_decode + c
        ops.append(("create",)); ops.append(("append", s, chunk_ctx))
        chunk_seqs.append(s)
    ops.append(("flush",))
    q = _normal(rng, (n_decode, hq, d), "bf16")
    chunk_q = _normal(rng, (n_chunks * chunk, hq, d), "bf16")
    total = n_decode * decode_ctx + n_chunks * chunk_ctx
    if with_rows:
        k_rows = _rows(rng, total, hkv, d, "bf16")
        v_rows = _rows(rng, total, hkv, d, "bf16")
    else:
        k_rows = v_rows = np.empty((0, hkv, d), dtype=np.uint16)
    qsl = np.arange(0, (n_chunks + 1) * chunk, chunk, dtype=np.int32)
    return Workload("long", "bf16", hq, hkv, d, need, perm, ops, k_rows, v_rows,
                    list(range(n_decode)), q, np.float32(1.0 / math.sqrt(d)),
                    chunk_seqs=chunk_seqs, chunk_q=chunk_q, chunk_query_start_loc=qsl)


def random_small(seed: int, num_seqs: int, max_ctx: int, hq: int, hkv: int, d: int,
                 dtype: str, pool_factor: float = 1.5, min_ctx: int = 1, block_size: int = BLOCK_SIZE) -> Workload:
    """A small ragged decode batch for parity tests (lengths uniform in [min_ctx, max_ctx])."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(min_ctx, max_ctx + 1, size=num_seqs).astype(np.int32)
    return _plain_decode(f"small{seed}", seed + 7919, ctx, hq, hkv, d, dtype,
                         pool_factor=pool_factor, block_size=block_size)


def from_lengths(seed: int, ctx, hq: int, hkv: int, d: int, dtype: str, pool_factor: float = 1.2,
                 block_size: int = BLOCK_SIZE) -> Workload:
    """A decode batch with the given context lengths (0 allowed)."""
    return _plain_decode(f"lengths{seed}", seed, ctx, hq, hkv, d, dtype, pool_factor=pool_factor,
                         block_size=block_size)


def random_prefill(seed: int, ctxs, n_queries, hq: int, hkv: int, d: int, pool_factor: float = 1.3,
                   block_size: int = BLOCK_SIZE, dtype: str = "bf16") -> Workload:
    """Chunked-prefill parity cases: sequence s has ctxs[s] cached tokens, the last
    n_queries[s] of which are its chunk's queries (bf16 or f32, the pool's
    type).  Every sequence also carries one decode query."""
    w = _plain_decode(f"prefill{seed}", seed + 104729, ctxs, hq, hkv, d, dtype, pool_factor=pool_factor,
                      block_size=block_size)
    rng = np.random.default_rng(seed + 31337)
    nq = np.asarray(n_queries, dtype=np.int32)
    w.chunk_seqs = list(range(len(ctxs)))
    w.chunk_q = _normal(rng, (int(nq.sum()), hq, d), dtype)
    w.chunk_query_start_loc = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    return w


@dataclasses.dataclass
class ServingWorkload:
    """Requests for a continuous-batching run.  Request r has prompts[r] prompt
    tokens and produces outputs[r] tokens; the cache ever holds positions
    0 .. prompts[r] + outputs[r] - 2 of it.  The K/V rows and the query of
    position p of request r are row ``row_start[r] + p`` of k_rows / v_rows /
    q_rows (a lookup table of inputs, nothing the method computes)."""
    name: str
    dtype: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    initial_free_order: np.ndarray
    num_host_blocks: int
    max_num_seqs: int
    max_num_batched_tokens: int
    prompts: np.ndarray           # int32 [R]
    outputs: np.ndarray           # int32 [R]
    row_start: np.ndarray         # int64 [R + 1]
    k_rows: np.ndarray            # [T, Hkv, d]
    v_rows: np.ndarray
    q_rows: np.ndarray            # [T, Hq, d]
    scale: np.float32
    block_size: int = BLOCK_SIZE


def serving(seed: int = 6, num_requests: int = 24, hq: int = 8, hkv: int = 2, d: int = 64,
            prompt_median: float = 40.0, output_median: float = 30.0, sigma: float = 0.8,
            max_prompt: int = 160, max_output: int = 96, num_blocks: int = 40,
            max_num_seqs: int = 8, max_num_batched_tokens: int = 256, num_host_blocks: int = 160,
            dtype: str = "bf16", with_rows: bool = True, block_size: int = BLOCK_SIZE) -> ServingWorkload:
    """A request stream for the continuous-batching loop: prompt and output
    lengths lognormal (the right-skewed mix of "Batching Continuo y
    PagedAttention", section on static batching), clipped to
    [1, max_prompt] / [1, max_output], each request's total clipped to what the
    device pool can hold; a device pool small enough that requests compete
    for blocks, so requests get swapped out to the host pool and back."""
    rng = np.random.default_rng(seed)
    prompts = lognormal_lengths(rng, num_requests, prompt_median, sigma, 1,
                                min(max_prompt, max_num_batched_tokens))
    outputs = lognormal_lengths(rng, num_requests, output_median, sigma, 1, max_output)
    cap = num_blocks * block_size
    outputs = np.minimum(outputs, cap - prompts).astype(np.int32)
    if np.any(outputs < 1):
        raise ValueError("device pool too small for the prompts drawn")
    perm = rng.permutation(num_blocks).astype(np.int32)
    per = (prompts + outputs - 1).astype(np.int64)
    row_start = np.concatenate([[0], np.cumsum(per)]).astype(np.int64)
    total = int(row_start[-1])
    if with_rows:
        k_rows = _rows(rng, total, hkv, d, dtype)
        v_rows = _rows(rng, total, hkv, d, dtype)
        q_rows = _rows(rng, total, hq, d, dtype)
    else:
        empty = np.empty((0, hkv, d), dtype=np.float32 if dtype == "f32" else np.uint16)
        k_rows = v_rows = empty
        q_rows = np.empty((0, hq, d), dtype=empty.dtype)
    return ServingWorkload(f"serving{seed}", dtype, hq, hkv, d, num_blocks, perm, num_host_blocks,
                           max_num_seqs, max_num_batched_tokens, prompts, outputs, row_start,
                           k_rows, v_rows, q_rows, np.float32(1.0 / math.sqrt(d)), block_size=block_size)


WORKLOADS = {1: tiny, 2: shaped_13b, 3: gqa, 4: parallel_sampling, 5: long_mix}
