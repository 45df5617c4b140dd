"""CPU oracle for paged KV-cache decode attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and its
Python binding) never calls it; the two share no code.

Everything here is plain, slow and written to be checked by eye against the
pages.  Floating point is carried in float64; storage values (fp32 or bf16
bits) are widened exactly.  Pages cited:

  [CB]  "Batching Continuo y PagedAttention" (cruxr.ai)
  [IPX] iplexlaw.co.kr commentary on the vLLM PagedAttention paper (arXiv v1)
  [OS]  "PagedAttention: gestionar la KV cache como memoria de un sistema
        operativo" (josueisai.com)
  [UL]  "Continuous Batching" (Ultralytics glossary)

Readings taken where the pages are silent (each also listed in the design notes):
  * attention is standard scaled dot-product softmax attention with a
    caller-supplied scale (the pages only say "scores per block, then a
    softmax-weighted sum");
  * a query head h reads KV head h // (Hq / Hkv) (contiguous groups);
  * a slot is ``block * block_size + offset`` and a slot of -1 is skipped;
  * free blocks are handed out first-in first-out, freed blocks go to the back
    in block-table order;
  * copy-on-write copies only a *partially filled* shared last block, at the
    first append into it; a *full* shared last block stays shared and the
    append starts a fresh block;
  * ctx = 0 gives an all-zero output row.
"""
from __future__ import annotations

import collections
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BLOCK_SIZE = 16


class OutOfBlocks(Exception):
    pass


class UnknownSequence(Exception):
    pass


# ---------------------------------------------------------------------------
# Block allocator model.
# [CB] "PagedAttention: Memoria virtual para la KV cache": each request keeps a
# page table from logical block i (tokens 16i..16i+15) to a physical block; a
# request gets a block when first scheduled, a new block from the free pool when
# its last one fills, and returns all blocks to the pool when it finishes.
# [OS] "Cómo funciona por dentro": a new block is requested only when the last
# one is full, from wherever a free block is.
# [IPX] "Dos respuestas a una entrada": tables of two answers may point at the
# same prompt blocks; a shared block that still has room is copied on write
# while other references exist; full shared blocks stay shared; blocks with no
# references are freed.  [CB] same section: copy-on-write sharing works like
# Unix fork().
# ---------------------------------------------------------------------------
class BlockAllocatorModel:
    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE,
                 initial_free_order: Optional[Sequence[int]] = None):
        if initial_free_order is None:
            initial_free_order = range(num_blocks)
        order = [int(b) for b in initial_free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("initial_free_order must be a permutation of range(num_blocks)")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free: collections.deque = collections.deque(order)
        self.ref: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        self.next_id = 0

    @property
    def num_free(self) -> int:
        return len(self.free)

    def create(self) -> int:
        sid = self.next_id
        self.next_id += 1
        self.tables[sid] = []
        self.lens[sid] = 0
        return sid

    def _check(self, sid: int) -> None:
        if sid not in self.tables:
            raise UnknownSequence(sid)

    def blocks_needed(self, sid: int, n: int) -> int:
        """Free blocks that append_slots(sid, n) would take."""
        self._check(sid)
        table, length = self.tables[sid], self.lens[sid]
        need = 0
        for i in range(n):
            pos = length + i
            if pos % self.block_size == 0:
                need += 1
            elif i == 0 and self.ref[table[-1]] > 1:
                need += 1
        return need

    def append_slots(self, sid: int, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Reserve slots for n new tokens; returns (slots, copy-on-write pairs).

        Raises OutOfBlocks without changing any state when the pool is short.
        """
        if n < 0:
            raise ValueError("n must be >= 0")
        if self.blocks_needed(sid, n) > len(self.free):
            raise OutOfBlocks(sid)
        table = self.tables[sid]
        slots: List[int] = []
        pairs: List[Tuple[int, int]] = []
        for _ in range(n):
            length = self.lens[sid]
            offset = length % self.block_size
            if offset == 0:
                # last block full (or no block yet): take the next free block
                b = self.free.popleft()
                self.ref[b] = 1
                table.append(b)
            elif self.ref[table[-1]] > 1:
                # writing into a shared, partially filled block: copy it first
                old = table[-1]
                b = self.free.popleft()
                self.ref[old] -= 1
                self.ref[b] = 1
                table[-1] = b
                pairs.append((old, b))
            slots.append(table[-1] * self.block_size + offset)
            self.lens[sid] = length + 1
        return slots, pairs

    def fork(self, parent: int) -> int:
        self._check(parent)
        child = self.create()
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1
        return child

    def free_seq(self, sid: int) -> None:
        self._check(sid)
        for b in self.tables[sid]:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.tables[sid]
        del self.lens[sid]

    def block_table(self, sid: int) -> List[int]:
        self._check(sid)
        return list(self.tables[sid])

    def num_tokens(self, sid: int) -> int:
        self._check(sid)
        return self.lens[sid]

    def refcount(self, block: int) -> int:
        return self.ref[block]


# ---------------------------------------------------------------------------
# Pool writes and block copies, on raw storage bits.
# Pool layout: [num_blocks][num_kv_heads][block_size][head_dim].
# [OS] "Cómo funciona por dentro": the new token's key and value go into the
# last block of the sequence's table.  [IPX] "Dos respuestas a una entrada":
# copy-on-write gives the writer its own copy of the shared block.
# ---------------------------------------------------------------------------
def _bits(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.float32:
        return a.view(np.uint32)
    if a.dtype == np.uint16:
        return a
    raise TypeError(f"unsupported storage dtype {a.dtype}")


def write_cache(k_pool: np.ndarray, v_pool: np.ndarray, k: np.ndarray, v: np.ndarray,
                slot_mapping: Sequence[int], block_size: int = BLOCK_SIZE) -> None:
    """pool[slot // P, h, slot % P, :] = row[t, h, :] for every t with slot >= 0 (in place)."""
    kp, vp, kb, vb = _bits(k_pool), _bits(v_pool), _bits(k), _bits(v)
    seen = set()
    for t, slot in enumerate(slot_mapping):
        slot = int(slot)
        if slot < 0:
            continue
        if slot in seen:
            raise ValueError(f"slot {slot} written twice in one call")
        seen.add(slot)
        blk, off = divmod(slot, block_size)
        kp[blk, :, off, :] = kb[t]
        vp[blk, :, off, :] = vb[t]


def copy_blocks(k_pool: np.ndarray, v_pool: np.ndarray, pairs: Sequence[Tuple[int, int]]) -> None:
    """pool[dst] = pool[src] for every pair, all reading the pool as it was before the call."""
    pairs = [(int(s), int(d)) for s, d in pairs]
    dsts = [d for _, d in pairs]
    if len(set(dsts)) != len(dsts) or set(dsts) & {s for s, _ in pairs}:
        raise ValueError("copy destinations must be distinct and not among the sources")
    for pool in (_bits(k_pool), _bits(v_pool)):
        before = {s: pool[s].copy() for s, _ in pairs}
        for s, d in pairs:
            pool[d] = before[s]


def swap_blocks(dst_k: np.ndarray, dst_v: np.ndarray, src_k: np.ndarray, src_v: np.ndarray,
                pairs: Sequence[Tuple[int, int]]) -> None:
    """dst[d] = src[s] between two pools (a swap to or from CPU memory).

    [CB] "Juntándolo todo: Arquitectura de vLLM": a preempted request's KV
    blocks are copied out to CPU memory and their GPU blocks freed; when memory
    is available they are copied back and the request resumes.  Whole blocks,
    bit for bit; destinations distinct."""
    pairs = [(int(s), int(d)) for s, d in pairs]
    dsts = [d for _, d in pairs]
    if len(set(dsts)) != len(dsts):
        raise ValueError("swap destinations must be distinct")
    for dst, src in ((_bits(dst_k), _bits(src_k)), (_bits(dst_v), _bits(src_v))):
        for s, d in pairs:
            dst[d] = src[s]


# ---------------------------------------------------------------------------
# Attention.
# [OS] "Cómo funciona por dentro": attention walks the sequence's blocks in
# table order, scores the query against each block's keys, then takes one
# softmax-weighted sum of the values.  [IPX] "Separar orden lógico y ubicación
# física": attention follows the logical order through the table; paging drops
# no token ("Gestión de memoria y documentación técnica").  So the result is
# exactly contiguous softmax attention over the gathered context.
# ---------------------------------------------------------------------------
def storage_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of fp32 values or bf16 bits (uint16) to float64."""
    if a.dtype == np.float32:
        return a.astype(np.float64)
    if a.dtype == np.uint16:
        f32 = (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
        return f32.astype(np.float64)
    raise TypeError(f"unsupported storage dtype {a.dtype}")


def gather_context(pool: np.ndarray, table: Sequence[int], ctx: int,
                   block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Rows of tokens 0..ctx-1 in logical order: [ctx, Hkv, d] storage values."""
    t = np.arange(ctx)
    blocks = np.asarray(table, dtype=np.int64)[t // block_size]
    return pool[blocks, :, t % block_size, :]


def kv_head_of(h: int, num_heads: int, num_kv_heads: int) -> int:
    return h // (num_heads // num_kv_heads)


def softmax_attention(qv: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * keys @ qv) @ values, in float64.  keys/values [n, d]; n >= 1."""
    z = scale * (keys @ qv)
    w = np.exp(z - z.max())
    return (w @ values) / w.sum()


def decode_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                     block_tables: Sequence[Sequence[int]], context_lens: Sequence[int],
                     scale, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """One query per sequence and head over that sequence's paged context -> float64 [S, Hq, d]."""
    S, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    scale64 = float(np.float32(scale))
    out = np.zeros((S, Hq, d), dtype=np.float64)
    for s in range(S):
        ctx = int(context_lens[s])
        if ctx == 0:
            continue
        K = storage_to_f64(gather_context(k_pool, block_tables[s], ctx, block_size))
        V = storage_to_f64(gather_context(v_pool, block_tables[s], ctx, block_size))
        qs = storage_to_f64(q[s])
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            out[s, h] = softmax_attention(qs[h], K[:, g, :], V[:, g, :], scale64)
    return out


def prefill_chunk_attention(q: np.ndarray, query_start_loc: Sequence[int], k_pool: np.ndarray,
                            v_pool: np.ndarray, block_tables: Sequence[Sequence[int]],
                            context_lens: Sequence[int], scale,
                            block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Causal attention of a prefill chunk that ends its sequence's context.

    [UL] "Cómo funciona la planificación a nivel de iteración" and "Límites y
    técnicas complementarias": long prompts are prefetched in chunks that run in
    the same step as other sequences' decode.  Sequence s owns queries
    query_start_loc[s] .. query_start_loc[s+1]-1; with n_s of them, query i sits
    at absolute position p_i = ctx_s - n_s + i and attends keys 0..p_i.
    Returns float64 [Tq, Hq, d].
    """
    Tq, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    scale64 = float(np.float32(scale))
    out = np.zeros((Tq, Hq, d), dtype=np.float64)
    for s in range(len(query_start_loc) - 1):
        a, b = int(query_start_loc[s]), int(query_start_loc[s + 1])
        ctx = int(context_lens[s])
        n = b - a
        if n > ctx:
            raise ValueError("chunk longer than its context")
        if n == 0:
            continue
        K = storage_to_f64(gather_context(k_pool, block_tables[s], ctx, block_size))
        V = storage_to_f64(gather_context(v_pool, block_tables[s], ctx, block_size))
        Q = storage_to_f64(q[a:b])                                  # [n, Hq, d]
        pos = ctx - n + np.arange(n)                                # absolute position of each query
        visible = np.arange(ctx)[None, :] <= pos[:, None]           # [n, ctx]: key t seen by query i
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            # every query's scores against every key of the context, then the
            # keys after the query's own position taken out of its softmax
            z = scale64 * (Q[:, h, :] @ K[:, g, :].T)
            z = np.where(visible, z, -np.inf)
            w = np.exp(z - z.max(axis=1, keepdims=True))
            out[a:b, h] = (w @ V[:, g, :]) / w.sum(axis=1, keepdims=True)
    return out


# ---------------------------------------------------------------------------
# Split-context partials and their merge (log-sum-exp algebra of the softmax).
# For a token range R:  m = max z,  l = sum exp(z - m),  acc = sum exp(z - m) v.
# Merging ranges:  M = max m_p,  o = sum acc_p e^(m_p - M) / sum l_p e^(m_p - M).
# The pages do not discuss splitting a context; this is the identity that makes
# a split softmax equal the unsplit one.
# ---------------------------------------------------------------------------
def attention_partial(qv: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float):
    z = scale * (keys @ qv)
    m = z.max()
    w = np.exp(z - m)
    return m, w.sum(), w @ values


def merge_partials(ms: Sequence[float], ls: Sequence[float], accs: Sequence[np.ndarray]) -> np.ndarray:
    M = max(ms)
    num = sum(acc * math.exp(m - M) for m, acc in zip(ms, accs))
    den = sum(l * math.exp(m - M) for m, l in zip(ms, ls))
    return num / den


# ---------------------------------------------------------------------------
# Memory accounting from [CB]; used by the accounting checks only.
# ---------------------------------------------------------------------------
def kv_cache_bytes(layers: int, heads: int, head_dim: int, tokens: int, elem_bytes: int) -> int:
    """[CB] "El problema de fragmentación de la KV cache": keys and values (factor 2)
    for every layer, head and head-dim element of every cached token."""
    return 2 * layers * heads * head_dim * tokens * elem_bytes


def paged_slots_reserved(tokens: int, block_size: int = BLOCK_SIZE) -> int:
    """[CB] "PagedAttention: Memoria virtual para la KV cache": a request of
    L tokens holds ceil(L / P) blocks."""
    return -(-tokens // block_size) * block_size


def cow_saving_bytes(n_requests: int, shared_tokens: int, bytes_per_token: float) -> float:
    """[CB] same section: N requests sharing S prompt tokens keep one copy instead of N."""
    return n_requests * shared_tokens * bytes_per_token - shared_tokens * bytes_per_token


def static_padding_waste(mean_len: float, max_len: float) -> float:
    """[CB] "Por qué el batching estático desperdicia GPUs": a static batch pads every
    request to the longest; padding is N (L_max - L_mean) of N L_max token-steps."""
    return (max_len - mean_len) / max_len


def preallocation_waste(length: int, max_len: int) -> float:
    """[CB] "PagedAttention: Memoria virtual para la KV cache": a reservation of
    L_max slots used by L tokens leaves L_max - L of them empty."""
    return (max_len - length) / max_len


# ---------------------------------------------------------------------------
# Replaying a workload script (create / fork / append / flush) on the model.
# ---------------------------------------------------------------------------
class ReplayResult:
    def __init__(self):
        self.alloc: Optional[BlockAllocatorModel] = None
        self.k_pool: Optional[np.ndarray] = None
        self.v_pool: Optional[np.ndarray] = None
        self.slots: List[int] = []          # slot of every appended row, in row order
        self.cow_pairs: List[Tuple[int, int]] = []


def replay(ops, k_rows: np.ndarray, v_rows: np.ndarray, num_blocks: int, num_kv_heads: int,
           head_dim: int, initial_free_order=None, block_size: int = BLOCK_SIZE,
           pool_fill=None) -> ReplayResult:
    """Run an operation script on the allocator model and the pool model.

    At each flush the pending block copies are applied first, then the pending
    row writes, so a copy reads its source as it was before this step's writes.
    ``pool_fill`` is the initial pool content (0 when None; may be NaN).
    """
    dtype = k_rows.dtype
    r = ReplayResult()
    r.alloc = BlockAllocatorModel(num_blocks, block_size, initial_free_order)
    shape = (num_blocks, num_kv_heads, block_size, head_dim)
    if pool_fill is None:
        r.k_pool = np.zeros(shape, dtype=dtype)
    else:
        r.k_pool = np.full(shape, pool_fill, dtype=dtype)
    r.v_pool = r.k_pool.copy()
    row = 0
    pend_rows: List[int] = []
    pend_slots: List[int] = []
    pend_pairs: List[Tuple[int, int]] = []
    for op in ops:
        if op[0] == "create":
            r.alloc.create()
        elif op[0] == "fork":
            r.alloc.fork(op[1])
        elif op[0] == "append":
            slots, pairs = r.alloc.append_slots(op[1], op[2])
            pend_rows.extend(range(row, row + op[2]))
            pend_slots.extend(slots)
            pend_pairs.extend(pairs)
            r.slots.extend(slots)
            r.cow_pairs.extend(pairs)
            row += op[2]
        elif op[0] == "flush":
            if pend_pairs:
                copy_blocks(r.k_pool, r.v_pool, pend_pairs)
            if pend_rows:
                idx = np.asarray(pend_rows)
                write_cache(r.k_pool, r.v_pool, k_rows[idx], v_rows[idx], pend_slots, block_size)
            pend_rows, pend_slots, pend_pairs = [], [], []
        else:
            raise ValueError(f"unknown op {op!r}")
    return r
