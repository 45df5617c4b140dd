"""Oracle of the continuous-batching loop on real data -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module.  It strings together, per scheduler step, the
oracle pieces the pages describe:

  [CB] "Juntándolo todo: Arquitectura de vLLM": each step the scheduler picks
       the requests to run, a swapped-out request's blocks are copied to CPU
       memory and back; the new tokens' K/V rows are written into their slots;
       attention then runs over each request's paged context.
  [UL] "Cómo funciona la planificación a nivel de iteración": newly admitted
       requests are prefilled in the same step in which the others decode.

Per step, in this order: swap-out copies (device -> host pool, reading the
device pool as the previous step left it), swap-in copies (host -> device),
the step's K/V rows into their slots, then causal prefill attention of every
admitted prompt over itself and decode attention of every decoding request
over its whole cached context (its newest token included).  The row of
position p of request r is the workload's row for (r, p).
"""
from __future__ import annotations

import dataclasses
from typing import List

import numpy as np

from .pkv_oracle import (BlockAllocatorModel, decode_attention, prefill_chunk_attention, swap_blocks,
                         write_cache)
from .scheduler import SchedulerModel, Step


@dataclasses.dataclass
class ServedStep:
    step: Step
    prefill_out: np.ndarray       # float64 [sum(prefill_lens), Hq, d]
    decode_out: np.ndarray        # float64 [len(decode), Hq, d]
    decode_positions: List[int]   # position of each decoding request's new token


class ServingModel:
    def __init__(self, w, policy: int):
        self.w = w
        shape = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
        hshape = (w.num_host_blocks,) + shape[1:]
        self.k_pool = np.zeros(shape, dtype=w.k_rows.dtype)
        self.v_pool = np.zeros(shape, dtype=w.k_rows.dtype)
        self.k_host = np.zeros(hshape, dtype=w.k_rows.dtype)
        self.v_host = np.zeros(hshape, dtype=w.k_rows.dtype)
        self.alloc = BlockAllocatorModel(w.num_blocks, w.block_size, w.initial_free_order)
        self.sched = SchedulerModel(self.alloc, w.max_num_seqs, w.max_num_batched_tokens, policy,
                                    w.num_host_blocks)
        for p, o in zip(w.prompts, w.outputs):
            self.sched.add_request(int(p), int(o))

    def _row(self, rid: int, pos: int) -> int:
        return int(self.w.row_start[rid]) + pos

    def step(self) -> ServedStep:
        w, sched = self.w, self.sched
        st = sched.step()
        if st.swap_out_pairs:
            swap_blocks(self.k_host, self.v_host, self.k_pool, self.v_pool, st.swap_out_pairs)
        if st.swap_in_pairs:
            swap_blocks(self.k_pool, self.v_pool, self.k_host, self.v_host, st.swap_in_pairs)
        rows = []
        for rid, n in zip(st.prefill, st.prefill_lens):
            rows += [self._row(rid, p) for p in range(n)]
        positions = []
        for rid in st.decode:
            pos = self.alloc.num_tokens(sched.requests[rid].seq) - 1
            positions.append(pos)
            rows.append(self._row(rid, pos))
        if rows:
            idx = np.asarray(rows)
            write_cache(self.k_pool, self.v_pool, w.k_rows[idx], w.v_rows[idx], st.slots, w.block_size)
        Hq, d = w.num_heads, w.head_dim
        n_pre = sum(st.prefill_lens)
        prefill_out = np.zeros((n_pre, Hq, d))
        if st.prefill:
            qidx = np.asarray([self._row(rid, p) for rid, n in zip(st.prefill, st.prefill_lens)
                               for p in range(n)])
            qsl = np.concatenate([[0], np.cumsum(st.prefill_lens)])
            tables = [self.alloc.block_table(sched.requests[r].seq) for r in st.prefill]
            prefill_out = prefill_chunk_attention(w.q_rows[qidx], qsl, self.k_pool, self.v_pool, tables,
                                                  st.prefill_lens, w.scale, w.block_size)
        decode_out = np.zeros((len(st.decode), Hq, d))
        if st.decode:
            qidx = np.asarray([self._row(r, p) for r, p in zip(st.decode, positions)])
            seqs = [sched.requests[r].seq for r in st.decode]
            decode_out = decode_attention(w.q_rows[qidx], self.k_pool, self.v_pool,
                                          [self.alloc.block_table(s) for s in seqs],
                                          [self.alloc.num_tokens(s) for s in seqs], w.scale, w.block_size)
        return ServedStep(st, prefill_out, decode_out, positions)
