"""Calls in flight at once: decode calls that split contexts (the merge ticket
and epoch inside the launch) and a chunked prefill enqueued on three streams
with nothing between them, and decode calls issued from two host threads at
the same time, each with its own stream and workspace.  Every output equals,
bit for bit, the same call run alone on one stream; those outputs are checked
against the oracle first.  Concurrent calls share no state in the library
beyond what each call is given (the workspace is per call and per stream)."""
import threading

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_kv_cache_171_amd as PK  # noqa: E402
import pkv_workloads as W  # noqa: E402
from oracle import pkv_oracle as O  # noqa: E402
from pkv_gpu_driver import GpuReplay, rows_to_device  # noqa: E402

TOL = 2e-3          # bf16 K/V

DECODES = [
    # seed, S, max_ctx, Hq, Hkv, d: contexts past 1024 tokens, so rows are merged in the launch
    (71, 9, 3300, 8, 8, 128),       # vector-ALU kernel (MHA)
    (72, 6, 9000, 16, 2, 128),      # matrix-core group kernel (GQA)
]


class _Decode:
    """One decode batch: its pools, tables and lengths on the device, the
    oracle's output, and a call on a given stream into a given output."""

    def __init__(self, seed, S, max_ctx, hq, hkv, d):
        w = W.random_small(seed, S, max_ctx, hq, hkv, d, "bf16")
        self.g = GpuReplay(w)
        r = O.replay(w.ops, w.k_rows, w.v_rows, w.num_blocks, w.num_kv_heads, w.head_dim, w.initial_free_order)
        tables, lens = self.g.tables(w.decode_seqs)
        assert int(lens.max()) > 1024
        self.ref = O.decode_attention(w.q, r.k_pool, r.v_pool, [r.alloc.block_table(s) for s in w.decode_seqs],
                                      [r.alloc.num_tokens(s) for s in w.decode_seqs], w.scale)
        self.q = rows_to_device(w.q, "cuda")
        self.td = torch.from_numpy(tables).cuda()
        self.ld = torch.from_numpy(lens).cuda()
        self.mcl = int(lens.max())
        self.shape = (S, hq, d)
        self.scale = float(w.scale)
        self.nws = PK.pkv_attention_workspace_bytes(S, hq, d, self.mcl)

    def workspace(self):
        return torch.empty(self.nws, dtype=torch.uint8, device="cuda")

    def call(self, out, ws, stream):
        PK.pkv_attention_decode(out, self.q, self.g.k_pool, self.g.v_pool, self.td, self.ld, self.mcl, self.scale,
                                workspace=ws, stream=stream)


class _Prefill:
    def __init__(self):
        w = W.random_prefill(73, [700, 1300, 90], [200, 129, 90], 16, 2, 128)
        self.g = GpuReplay(w)
        r = O.replay(w.ops, w.k_rows, w.v_rows, w.num_blocks, w.num_kv_heads, w.head_dim, w.initial_free_order)
        qsl = w.chunk_query_start_loc
        self.ref = O.prefill_chunk_attention(w.chunk_q, qsl, r.k_pool, r.v_pool,
                                             [r.alloc.block_table(s) for s in w.chunk_seqs],
                                             [r.alloc.num_tokens(s) for s in w.chunk_seqs], w.scale)
        tables, lens = self.g.tables(w.chunk_seqs)
        self.q = rows_to_device(w.chunk_q, "cuda")
        self.qsl = torch.from_numpy(qsl.astype(np.int32)).cuda()
        self.mql = int(np.max(np.diff(qsl)))
        self.td = torch.from_numpy(tables).cuda()
        self.ld = torch.from_numpy(lens).cuda()
        self.mcl = int(lens.max())
        self.shape = (int(qsl[-1]), w.num_heads, w.head_dim)
        self.scale = float(w.scale)

    def call(self, out, stream):
        PK.pkv_attention_prefill_chunk(out, self.q, self.qsl, self.mql, self.g.k_pool, self.g.v_pool, self.td,
                                       self.ld, self.mcl, self.scale, stream=stream)


def _empty(shape):
    return torch.full(shape, -7.0, dtype=torch.float32, device="cuda")


def test_calls_on_three_streams_at_once_give_the_bits_of_one_stream():
    print("case: two split-context decodes and a prefill on three streams, 3 rounds", flush=True)
    decs = [_Decode(*c) for c in DECODES]
    pre = _Prefill()
    main = torch.cuda.current_stream()
    # each call alone, in turn, on one stream
    alone = []
    for dc in decs:
        out = _empty(dc.shape)
        dc.call(out, dc.workspace(), main)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert float(np.abs(got - dc.ref).max()) <= TOL
        alone.append(got)
    out = _empty(pre.shape)
    pre.call(out, main)
    torch.cuda.synchronize()
    pre_alone = out.cpu().numpy()
    assert float(np.abs(pre_alone - pre.ref).max()) <= TOL

    # the same calls, three rounds of each, on three streams with nothing between them
    streams = [torch.cuda.Stream() for _ in range(3)]
    start = torch.cuda.Event()
    start.record(main)
    for s in streams:
        s.wait_event(start)
    rounds = 3
    wss = [dc.workspace() for dc in decs]                    # one workspace per stream
    outs = [[_empty(dc.shape) for _ in range(rounds)] for dc in decs]
    pouts = [_empty(pre.shape) for _ in range(rounds)]
    for k in range(rounds):
        for i, dc in enumerate(decs):
            dc.call(outs[i][k], wss[i], streams[i])
        pre.call(pouts[k], streams[2])
    for s in streams:
        done = torch.cuda.Event()
        done.record(s)
        main.wait_event(done)
    torch.cuda.synchronize()
    for i in range(len(decs)):
        for k in range(rounds):
            assert np.array_equal(outs[i][k].cpu().numpy(), alone[i]), (i, k)
    for k in range(rounds):
        assert np.array_equal(pouts[k].cpu().numpy(), pre_alone), k


def test_decode_from_two_host_threads_at_once():
    print("case: two host threads, each 8 split-context decodes on its own stream", flush=True)
    decs = [_Decode(*c) for c in DECODES]
    main = torch.cuda.current_stream()
    alone = []
    for dc in decs:
        out = _empty(dc.shape)
        dc.call(out, dc.workspace(), main)
        torch.cuda.synchronize()
        alone.append(out.cpu().numpy())
    calls = 8
    outs = [[_empty(dc.shape) for _ in range(calls)] for dc in decs]
    wss = [dc.workspace() for dc in decs]
    streams = [torch.cuda.Stream() for _ in decs]
    errors = []
    barrier = threading.Barrier(len(decs))

    def work(i):
        try:
            torch.cuda.set_device(0)
            barrier.wait()
            for k in range(calls):
                decs[i].call(outs[i][k], wss[i], streams[i])
            streams[i].synchronize()
        except Exception as e:  # reported by the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(decs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a decode thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(len(decs)):
        for k in range(calls):
            assert np.array_equal(outs[i][k].cpu().numpy(), alone[i]), (i, k)
