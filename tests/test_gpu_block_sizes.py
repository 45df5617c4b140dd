"""Block sizes 8 and 32 (the 16 of the pages is covered everywhere else) through
the C ABI against the oracle: allocator tables, slots, copy-on-write pairs and
whole pools bit-exact after copy + append; decode attention (fp32 within 1e-5,
bf16 within 2e-3) for MHA (vector-ALU kernel) and grouped-query heads (the
matrix-core kernel, which walks contexts in 16-key tiles: two 8-token blocks
or half a 32-token block per tile), planned decode, a plan built for another
block size, swap copies, shared-prefix decode (plain and planned) and causal
chunked prefill at these sizes."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_kv_cache_171_amd as PK  # noqa: E402
import pkv_workloads as W  # noqa: E402
from oracle import pkv_oracle as O  # noqa: E402
from pkv_gpu_driver import GpuReplay, pool_to_host, rows_to_device  # noqa: E402

TOL = {"f32": 1e-5, "bf16": 2e-3}


def _oracle(w):
    return O.replay(w.ops, w.k_rows, w.v_rows, w.num_blocks, w.num_kv_heads, w.head_dim, w.initial_free_order,
                    block_size=w.block_size)


def _check(w, planned=False):
    g, r = GpuReplay(w), _oracle(w)
    assert g.slots == r.slots and [tuple(p) for p in g.cow_pairs] == r.cow_pairs
    assert np.array_equal(pool_to_host(g.k_pool), r.k_pool) and np.array_equal(pool_to_host(g.v_pool), r.v_pool)
    tables, lens = g.tables(w.decode_seqs)
    for i, s in enumerate(w.decode_seqs):
        assert list(tables[i, :len(r.alloc.block_table(s))]) == r.alloc.block_table(s)
    mcl = int(lens.max())
    qd = rows_to_device(w.q, "cuda")
    td, ld = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()
    out = torch.full((len(w.decode_seqs), w.num_heads, w.head_dim), -3.0, dtype=torch.float32, device="cuda")
    plan = None
    if planned:
        plan = PK.plan_for(ld, w.num_heads, w.num_kv_heads, tables.shape[1], mcl,
                           PK.PKV_BF16 if w.dtype == "bf16" else PK.PKV_F32, block_size=w.block_size)
    PK.pkv_attention_decode(out, qd, g.k_pool, g.v_pool, td, ld, mcl, float(w.scale), plan=plan)
    torch.cuda.synchronize()
    ref = O.decode_attention(w.q, r.k_pool, r.v_pool, [r.alloc.block_table(s) for s in w.decode_seqs],
                             [r.alloc.num_tokens(s) for s in w.decode_seqs], w.scale, block_size=w.block_size)
    err = float(np.abs(out.cpu().numpy() - ref).max())
    assert err <= TOL[w.dtype], err
    return g, qd, td, ld, mcl


@pytest.mark.parametrize("bs", [8, 32])
@pytest.mark.parametrize("dtype,hq,hkv,d,max_ctx", [("f32", 4, 4, 64, 700), ("f32", 8, 2, 128, 2100),
                                                    ("bf16", 8, 8, 128, 2500), ("bf16", 16, 2, 64, 1500),
                                                    ("bf16", 32, 8, 128, 900), ("bf16", 16, 2, 128, 9000),
                                                    ("bf16", 8, 4, 128, 77), ("bf16", 48, 1, 64, 2100),
                                                    ("bf16", 64, 2, 128, 1300), ("f32", 48, 1, 64, 2100),
                                                    ("f32", 32, 1, 128, 1300)])
def test_decode_and_cache_ops(bs, dtype, hq, hkv, d, max_ctx):
    print(f"case: bs={bs} {dtype} {hq}/{hkv} d={d} ctx<={max_ctx}", flush=True)
    w = W.random_small(100 + bs, 9, max_ctx, hq, hkv, d, dtype, block_size=bs)
    _check(w)
    _check(w, planned=True)


@pytest.mark.parametrize("bs", [8, 32])
def test_forks_copy_on_write(bs):
    print(f"case: bs={bs} forks", flush=True)
    w = W.parallel_sampling(seed=30 + bs, groups=3, samples=[4, 2, 3], prompt=[77, 40, 130], tail_lo=0, tail_hi=60,
                            hq=8, d=128, block_size=bs)
    _check(w)


def test_a_plan_for_another_block_size_gives_nan_rows():
    print("case: bs plan mismatch", flush=True)
    w = W.random_small(7, 5, 300, 4, 4, 64, "f32", block_size=8)
    g, qd, td, ld, mcl = _check(w)
    plan = PK.plan_for(ld, 4, 4, td.shape[1], mcl, PK.PKV_F32, block_size=16)
    out = torch.zeros((5, 4, 64), dtype=torch.float32, device="cuda")
    PK.pkv_attention_decode(out, qd, g.k_pool, g.v_pool, td, ld, mcl, float(w.scale), plan=plan)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()


@pytest.mark.parametrize("bs", [8, 32])
def test_swap_copies(bs):
    print(f"case: bs={bs} swap", flush=True)
    rng = np.random.default_rng(bs)
    dk = rng.integers(0, 1 << 16, (12, 2, bs, 64), dtype=np.uint16)
    dv = rng.integers(0, 1 << 16, (12, 2, bs, 64), dtype=np.uint16)
    hk = np.zeros((7, 2, bs, 64), dtype=np.uint16)
    hv = np.zeros_like(hk)
    gdk, gdv = rows_to_device(dk, "cuda"), rows_to_device(dv, "cuda")
    ghk, ghv = rows_to_device(hk, "cpu").pin_memory(), rows_to_device(hv, "cpu").pin_memory()
    pairs = [(3, 0), (11, 6), (0, 2)]
    PK.pkv_swap_blocks(ghk, ghv, gdk, gdv, torch.tensor(pairs, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    O.swap_blocks(hk, hv, dk, dv, pairs)
    assert np.array_equal(pool_to_host(ghk), hk) and np.array_equal(pool_to_host(ghv), hv)


@pytest.mark.parametrize("bs", [8, 32])
@pytest.mark.parametrize("hq,hkv,d,dtype", [(8, 8, 128, "bf16"), (16, 2, 128, "bf16"), (4, 4, 64, "bf16"),
                                            (8, 8, 128, "f32"), (16, 2, 64, "f32")])
def test_shared_prefix_decode(bs, hq, hkv, d, dtype):
    """The groups' common leading blocks read once on the matrix cores (with
    8-token blocks an odd last common block is left to the members' own
    units): the oracle's result, and planned calls give the same bits."""
    print(f"case: bs={bs} shared {hq}/{hkv} d={d} {dtype}", flush=True)
    w = W.parallel_sampling(seed=41 + bs, groups=3, samples=[5, 2, 8], prompt=[70, 1100, 200], tail_lo=0,
                            tail_hi=50, hq=hq, hkv=hkv, d=d, block_size=bs, dtype=dtype)
    g, qd, td, ld, mcl = _check(w)
    r = _oracle(w)
    S = len(w.decode_seqs)
    gs = torch.tensor(w.group_start, dtype=torch.int32, device="cuda")
    out = torch.full((S, hq, d), -1.0, dtype=torch.float32, device="cuda")
    PK.pkv_attention_decode_shared(out, qd, g.k_pool, g.v_pool, td, ld, gs, mcl, float(w.scale))
    plan = PK.shared_plan_for(td, ld, gs, hq, hkv, mcl, PK.PKV_BF16 if dtype == "bf16" else PK.PKV_F32,
                              block_size=bs)
    out2 = torch.full_like(out, -2.0)
    PK.pkv_attention_decode_shared_planned(out2, qd, g.k_pool, g.v_pool, td, ld, mcl, float(w.scale), plan)
    torch.cuda.synchronize()
    ref = O.decode_attention(w.q, r.k_pool, r.v_pool, [r.alloc.block_table(s) for s in w.decode_seqs],
                             [r.alloc.num_tokens(s) for s in w.decode_seqs], w.scale, block_size=bs)
    assert float(np.abs(out.cpu().numpy() - ref).max()) <= TOL[dtype]
    assert torch.equal(out, out2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("bs", [8, 32])
@pytest.mark.parametrize("ctxs,nqs,hq,hkv,d", [
    ([60, 300, 700], [37, 64, 100], 8, 2, 128),
    ([16, 33, 129, 1], [16, 1, 129, 1], 4, 4, 64),
    ([1000, 45], [200, 5], 32, 1, 128),
])
def test_chunked_prefill(bs, ctxs, nqs, hq, hkv, d, dtype):
    """Causal chunked prefill with 8- or 32-token blocks (a 32-key pair of the
    bf16 kernel is four 8-token blocks or one 32-token block, a 16-key tile of
    the float32 kernel two 8-token blocks or half a 32-token block), every
    query row against the oracle."""
    print(f"case: bs={bs} prefill {dtype} ctx={ctxs} n={nqs} H={hq}/{hkv} d={d}", flush=True)
    w = W.random_prefill(90 + bs, ctxs, nqs, hq, hkv, d, block_size=bs, dtype=dtype)
    g, r = GpuReplay(w), _oracle(w)
    out, _, _ = g.prefill()
    tables = [r.alloc.block_table(s) for s in w.chunk_seqs]
    lens = [r.alloc.num_tokens(s) for s in w.chunk_seqs]
    ref = O.prefill_chunk_attention(w.chunk_q, w.chunk_query_start_loc, r.k_pool, r.v_pool, tables, lens, w.scale,
                                    block_size=bs)
    assert np.isfinite(out).all()
    assert float(np.abs(out - ref).max()) <= TOL[dtype]
