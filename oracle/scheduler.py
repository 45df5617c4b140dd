"""Oracle model of iteration-level (continuous) batching -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module; the native scheduler in the HIP library shares no
code with it.  Plain Python, written to be read against the pages:

  [UL] "Continuous Batching" (Ultralytics glossary), "Cómo funciona la
       planificación a nivel de iteración": after every decode step the
       scheduler returns finished sequences, frees their memory and admits
       queued requests if they fit in the KV cache; a new request is prefilled
       in the same step in which the others decode.  Its slot simulation: static
       batching keeps a group of requests together until the longest finishes;
       continuous batching gives a freed slot to the next request at once.
       "Límites y técnicas complementarias": engines cap the sequences and the
       tokens of a step (max_num_seqs, max_num_batched_tokens).
  [CB] "Batching Continuo y PagedAttention" (cruxr.ai), "Juntándolo todo:
       Arquitectura de vLLM": admission needs enough free KV blocks; a running
       request gets a new block when its last one is full; on finish all its
       blocks return to the pool; under memory pressure a low-priority request is
       swapped out -- its blocks copied to CPU memory and freed on the GPU -- and
       copied back to resume where it stopped once memory is available.

Readings where the pages are silent (also listed in the design notes):
  * a request of output length L occupies its slot for L steps: the step that
    admits it prefills its prompt and yields its first token, each of the next
    L - 1 steps decodes one more (the cache holds prompt + L - 1 tokens at the
    end); it finishes, and its blocks are freed, at the start of the next step;
  * order inside a step: finished requests leave; running requests reserve
    their decode slot in admission order, swapping out the most recently
    admitted running request (its whole table, to host blocks taken first in
    first out) while the pool is short (with no host space left, that request
    and the ones after it wait a step); if nothing was swapped out this step,
    swapped requests come back first in first out (a new table of fresh blocks,
    one host -> device copy per block, then their decode slot); then queued
    requests are admitted first in first out while a sequence slot, the token
    budget and free blocks for the whole prompt allow; a waiting request never
    passes a swapped one;
  * static batching admits a new group only when no request is running or
    swapped;
  * slots of a step: prefill tokens of the admitted requests (admission order),
    then one decode token per decoding request (reservation order).
"""
from __future__ import annotations

import collections
import dataclasses
from typing import List, Optional, Tuple

from .pkv_oracle import BLOCK_SIZE, BlockAllocatorModel

CONTINUOUS, STATIC = 0, 1
WAITING, RUNNING, SWAPPED, FINISHED = 0, 1, 2, 3


@dataclasses.dataclass
class Request:
    rid: int
    prompt: int
    output: int
    generated: int = 0
    seq: Optional[int] = None
    state: int = WAITING
    host_table: List[int] = dataclasses.field(default_factory=list)
    length: int = 0          # tokens in the cache while swapped


@dataclasses.dataclass
class Step:
    finished: List[int]
    swapped_out: List[int]
    swap_out_pairs: List[Tuple[int, int]]     # (device block, host block)
    swapped_in: List[int]
    swap_in_pairs: List[Tuple[int, int]]      # (host block, device block)
    prefill: List[int]
    prefill_lens: List[int]
    decode: List[int]
    slots: List[int]


class SchedulerModel:
    def __init__(self, alloc: BlockAllocatorModel, max_num_seqs: int, max_num_batched_tokens: int,
                 policy: int = CONTINUOUS, num_host_blocks: int = 0):
        self.alloc = alloc
        self.max_num_seqs = max_num_seqs
        self.max_tokens = max_num_batched_tokens
        self.policy = policy
        self.requests: List[Request] = []
        self.queue: collections.deque = collections.deque()
        self.running: List[Request] = []
        self.swapped: collections.deque = collections.deque()
        self.host_free: collections.deque = collections.deque(range(num_host_blocks))
        self.steps = 0
        self.busy = 0
        self.tokens = 0

    def add_request(self, prompt: int, output: int) -> int:
        # a request must fit the token budget and, at full length (+1 token of
        # headroom for a swap-in), the device pool
        if prompt < 1 or output < 1 or prompt > self.max_tokens or \
                self._fresh_blocks(prompt + output) > self.alloc.num_blocks:
            raise ValueError("request cannot ever be scheduled")
        r = Request(len(self.requests), prompt, output)
        self.requests.append(r)
        self.queue.append(r)
        return r.rid

    def done(self) -> bool:
        """No request is waiting, running or swapped (finished ones still
        running leave at the next step call, which then runs nothing)."""
        return not self.queue and not self.running and not self.swapped

    def _fresh_blocks(self, tokens: int) -> int:
        return -(-tokens // self.alloc.block_size)

    def _swap_out(self, r: Request, st: Step) -> bool:
        table = self.alloc.block_table(r.seq)
        if len(table) > len(self.host_free):
            return False
        host = [self.host_free.popleft() for _ in table]
        st.swap_out_pairs += list(zip(table, host))
        r.length = self.alloc.num_tokens(r.seq)
        self.alloc.free_seq(r.seq)
        r.seq = None
        r.host_table = host
        r.state = SWAPPED
        self.swapped.append(r)
        self.running.remove(r)
        st.swapped_out.append(r.rid)
        return True

    def step(self) -> Step:
        st = Step([], [], [], [], [], [], [], [], [])
        # 1. requests that produced all their tokens leave and free their blocks
        for r in list(self.running):
            if r.generated == r.output:
                self.alloc.free_seq(r.seq)
                r.seq = None
                r.state = FINISHED
                self.running.remove(r)
                st.finished.append(r.rid)
        if self.done():
            return st                      # the last requests left: no step runs
        budget = self.max_tokens
        decode_slots: List[int] = []
        # 2. running requests reserve one decode slot each; while the pool is
        #    short, the most recently admitted running request is swapped out
        #    (with no host space left, r and the requests after it wait a step)
        i = 0
        stalled = False
        while i < len(self.running):
            r = self.running[i]
            while self.alloc.blocks_needed(r.seq, 1) > self.alloc.num_free:
                if not self._swap_out(self.running[-1], st):
                    stalled = True
                    break
                if r.state == SWAPPED:
                    break
            if stalled or r.state != RUNNING:
                break                      # r itself went out: every later one went before it
            decode_slots += self.alloc.append_slots(r.seq, 1)[0]
            st.decode.append(r.rid)
            budget -= 1
            i += 1
        # 3. swapped requests return (not in a step that swapped out or stalled)
        if not st.swapped_out and not stalled:
            while self.swapped and len(self.running) < self.max_num_seqs and budget >= 1:
                r = self.swapped[0]
                need = self._fresh_blocks(r.length) + (1 if r.length % self.alloc.block_size == 0 else 0)
                if need > self.alloc.num_free:
                    break
                self.swapped.popleft()
                r.seq = self.alloc.create()
                self.alloc.append_slots(r.seq, r.length)
                table = self.alloc.block_table(r.seq)
                st.swap_in_pairs += list(zip(r.host_table, table))
                self.host_free.extend(r.host_table)
                r.host_table = []
                r.state = RUNNING
                self.running.append(r)
                st.swapped_in.append(r.rid)
                decode_slots += self.alloc.append_slots(r.seq, 1)[0]
                st.decode.append(r.rid)
                budget -= 1
        # 4. queued requests are admitted and prefilled
        prefill_slots: List[int] = []
        may_admit = not stalled and (self.policy == CONTINUOUS or (not self.running and not self.swapped))
        while may_admit and self.queue and not self.swapped and len(self.running) < self.max_num_seqs:
            r = self.queue[0]
            if r.prompt > budget or self._fresh_blocks(r.prompt) > self.alloc.num_free:
                break
            self.queue.popleft()
            r.seq = self.alloc.create()
            prefill_slots += self.alloc.append_slots(r.seq, r.prompt)[0]
            r.state = RUNNING
            self.running.append(r)
            st.prefill.append(r.rid)
            st.prefill_lens.append(r.prompt)
            budget -= r.prompt
        st.slots = prefill_slots + decode_slots
        # 5. every scheduled request yields one token
        for rid in st.prefill + st.decode:
            self.requests[rid].generated += 1
        n = len(st.prefill) + len(st.decode)
        if n == 0 and not self.done():
            raise RuntimeError("no request can make progress (host swap space exhausted)")
        self.steps += 1
        self.busy += n
        self.tokens += n
        return st
