"""The partition merge inside the decode launch: the last unit of a split row to
finish merges the row, counted on a ticket word in the workspace.

A workspace full of random bytes (tickets included) gives the oracle's result,
and calls that reuse it give the same bits; a decode captured in a HIP graph and
replayed (every replay reuses the captured launch's ticket epoch) matches the
eager call on every replay.  VALU kernel (MHA, bf16 and fp32) and MFMA group
kernel (GQA; batches this small take its 1024-token partitions); rows of up
to 40 partitions (the merge reads partials 8 at a time)."""
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

TOL = {"f32": 1e-5, "bf16": 2e-3}

CASES = [
    # seed, S, max_ctx, Hq, Hkv, d, dtype
    (61, 9, 3300, 8, 8, 128, "bf16"),     # VALU: up to 3 partitions of 1024
    (62, 7, 2600, 4, 4, 64, "f32"),
    (63, 5, 9000, 16, 2, 128, "bf16"),    # MFMA: up to 9 partitions
    (64, 3, 12000, 4, 4, 64, "f32"),      # VALU: 12 partitions, merged in two chunks of 8
    (66, 3, 40000, 8, 2, 64, "bf16"),     # MFMA: up to 40 partitions
    (67, 4, 13000, 8, 2, 128, "f32"),     # fp32 MFMA: up to 13 partitions
    (68, 3, 9000, 32, 1, 128, "bf16"),    # wide group kernel: two 16-row slices, each merged on its own ticket
    (69, 3, 9000, 48, 1, 64, "f32"),      # float32 wide group kernel: three slices
]


def _setup(seed, S, max_ctx, hq, hkv, d, dtype):
    w = W.random_small(seed, S, max_ctx, hq, hkv, d, dtype)
    g = GpuReplay(w)
    r = O.replay(w.ops, w.k_rows, w.v_rows, w.num_blocks, w.num_kv_heads, w.head_dim, w.initial_free_order)
    tables, lens = g.tables(w.decode_seqs)
    assert int(lens.max()) > 1024           # at least one row is merged in the launch
    ref = O.decode_attention(w.q, r.k_pool, r.v_pool, [r.alloc.block_table(s) for s in w.decode_seqs],
                             [r.alloc.num_tokens(s) for s in w.decode_seqs], w.scale)
    dev = dict(q=rows_to_device(w.q, "cuda"), td=torch.from_numpy(tables).cuda(),
               ld=torch.from_numpy(lens).cuda(), mcl=int(lens.max()))
    return w, g, ref, dev


@pytest.mark.parametrize("seed,S,max_ctx,hq,hkv,d,dtype", CASES)
def test_random_workspace_bytes_and_reuse(seed, S, max_ctx, hq, hkv, d, dtype):
    print(f"case: merge in launch, random workspace seed={seed} {hq}/{hkv} {dtype}", flush=True)
    w, g, ref, x = _setup(seed, S, max_ctx, hq, hkv, d, dtype)
    n = PK.pkv_attention_workspace_bytes(S, hq, d, x["mcl"])
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    ws = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=gen)
    results = []
    for _ in range(3):
        out = torch.full((S, hq, d), -3.0, dtype=torch.float32, device="cuda")
        PK.pkv_attention_decode(out, x["q"], g.k_pool, g.v_pool, x["td"], x["ld"], x["mcl"], float(w.scale),
                                workspace=ws)
        torch.cuda.synchronize()
        results.append(out.cpu().numpy())
    err = float(np.abs(results[0] - ref).max())
    assert err <= TOL[dtype], err
    assert np.array_equal(results[0], results[1]) and np.array_equal(results[0], results[2])


@pytest.mark.parametrize("seed,S,max_ctx,hq,hkv,d,dtype", [CASES[0], CASES[2], CASES[6], CASES[7]])
def test_graph_replays_match_the_eager_call(seed, S, max_ctx, hq, hkv, d, dtype):
    print(f"case: merge in launch, graph replay seed={seed} {hq}/{hkv} {dtype}", flush=True)
    w, g, ref, x = _setup(seed, S, max_ctx, hq, hkv, d, dtype)
    ws = PK.workspace_for(S, hq, d, x["mcl"])
    eager = torch.empty((S, hq, d), dtype=torch.float32, device="cuda")
    PK.pkv_attention_decode(eager, x["q"], g.k_pool, g.v_pool, x["td"], x["ld"], x["mcl"], float(w.scale),
                            workspace=ws)
    torch.cuda.synchronize()
    e = eager.cpu().numpy()
    assert float(np.abs(e - ref).max()) <= TOL[dtype]

    out = torch.full((S, hq, d), -3.0, dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        PK.pkv_attention_decode(out, x["q"], g.k_pool, g.v_pool, x["td"], x["ld"], x["mcl"], float(w.scale),
                                workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        PK.pkv_attention_decode(out, x["q"], g.k_pool, g.v_pool, x["td"], x["ld"], x["mcl"], float(w.scale),
                                workspace=ws)
    other = torch.empty_like(eager)
    for _ in range(4):
        out.fill_(-3.0)
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), e)
        # eager work on the same workspace between the replays
        PK.pkv_attention_decode(other, x["q"], g.k_pool, g.v_pool, x["td"], x["ld"], x["mcl"], float(w.scale),
                                workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(other.cpu().numpy(), e)


SHARED = [
    # seed, hq, hkv, d, samples, prompt, tail_lo, tail_hi, dtype: every row has
    # 2 or 3 prefix partials (prompts past 1024 tokens) plus its own
    (91, 8, 8, 128, [4, 3], [1500, 2100], 0, 40, "bf16"),       # MHA: vector-ALU own units
    (92, 32, 8, 128, [6, 2], [1100, 3000], 1, 1200, "bf16"),    # G=4: matrix-core own units, some split
    # float32: the shared units and the own units are two launches on one ticket epoch
    (93, 8, 8, 128, [4, 3], [1500, 2100], 0, 40, "f32"),
    (94, 32, 8, 128, [6, 2], [1100, 3000], 1, 1200, "f32"),
]


@pytest.mark.parametrize("seed,hq,hkv,d,samples,prompt,tail_lo,tail_hi,dtype", SHARED)
def test_shared_prefix_merge_with_random_workspace_and_graph_replays(seed, hq, hkv, d, samples, prompt,
                                                                      tail_lo, tail_hi, dtype):
    print(f"case: merge in launch, shared prefix seed={seed} {hq}/{hkv} {dtype}", flush=True)
    w = W.parallel_sampling(seed=seed, groups=len(samples), samples=samples, prompt=prompt, tail_lo=tail_lo,
                            tail_hi=tail_hi, hq=hq, hkv=hkv, d=d, dtype=dtype)
    g = GpuReplay(w)
    r = O.replay(w.ops, w.k_rows, w.v_rows, w.num_blocks, w.num_kv_heads, w.head_dim, w.initial_free_order)
    tables, lens = g.tables(w.decode_seqs)
    S, mcl = len(w.decode_seqs), int(lens.max())
    ref = O.decode_attention(w.q, r.k_pool, r.v_pool, [r.alloc.block_table(s) for s in w.decode_seqs],
                             [r.alloc.num_tokens(s) for s in w.decode_seqs], w.scale)
    q = rows_to_device(w.q, "cuda")
    td, ld = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()
    gs = torch.from_numpy(np.ascontiguousarray(w.group_start, dtype=np.int32)).cuda()
    n = PK.pkv_attention_decode_shared_workspace_bytes(S, hq, d, mcl)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    ws = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=gen)

    def call(out):
        PK.pkv_attention_decode_shared(out, q, g.k_pool, g.v_pool, td, ld, gs, mcl, float(w.scale), workspace=ws)

    eager = torch.full((S, hq, d), -3.0, dtype=torch.float32, device="cuda")
    call(eager)
    torch.cuda.synchronize()
    e = eager.cpu().numpy()
    err = float(np.abs(e - ref).max())
    assert err <= TOL[dtype], err
    out = torch.full_like(eager, -3.0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out)
    for _ in range(3):
        out.fill_(-3.0)
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), e)
        other = torch.full_like(eager, -3.0)
        call(other)
        torch.cuda.synchronize()
        assert np.array_equal(other.cpu().numpy(), e)
