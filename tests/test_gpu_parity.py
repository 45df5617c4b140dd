"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bit-exact: allocator tables, slots and copy pairs; pool contents after copy and
append (every byte, untouched ones included).  Attention: max abs error <= 1e-5
for fp32 K/V and <= 2e-3 for bf16 K/V against the float64 oracle, on every
workload at full size and on every output row (all decode rows of all five
workloads, every query of the long workload's prefill chunks), plus edge cases.
"""
import math

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


def _oracle(w, pool_fill=None):
    return O.replay(w.ops, w.k_rows, w.v_rows, w.num_blocks, w.num_kv_heads, w.head_dim,
                    w.initial_free_order, pool_fill=pool_fill)


def _check_state(g, r, w):
    assert g.slots == r.slots
    assert [tuple(p) for p in g.cow_pairs] == r.cow_pairs
    assert g.alloc.num_free == r.alloc.num_free
    for s in w.decode_seqs:
        t, n = g.alloc.seq_block_table(s)
        assert t == r.alloc.block_table(s) and n == r.alloc.num_tokens(s)
    assert np.array_equal(pool_to_host(g.k_pool), r.k_pool.view(r.k_pool.dtype))
    assert np.array_equal(pool_to_host(g.v_pool), r.v_pool)


def _attn_err(g, r, w):
    """Max abs error of every decode row of the workload against the oracle."""
    out, tables, lens = g.decode()
    ref = O.decode_attention(w.q, r.k_pool, r.v_pool, [r.alloc.block_table(s) for s in w.decode_seqs],
                             [r.alloc.num_tokens(s) for s in w.decode_seqs], w.scale)
    assert out.shape == ref.shape
    assert np.isfinite(out).all()
    return float(np.abs(out - ref).max())


_BIG = {}


def _big(name):
    """The full-size workload, its GPU replay and its oracle replay, built once
    per module (the long workload serves both its decode and its prefill test)."""
    if name not in _BIG:
        _BIG.clear()
        w = {"gqa": W.gqa, "fork": W.parallel_sampling, "long": W.long_mix}[name]()
        _BIG[name] = (w, GpuReplay(w), _oracle(w))
    return _BIG[name]


def test_tiny_workload_bit_exact_state_and_attention():
    w = W.tiny()
    print("case: tiny", flush=True)
    g, r = GpuReplay(w), _oracle(w)
    _check_state(g, r, w)
    err = _attn_err(g, r, w)
    assert err <= TOL["f32"], err


SMALL = [
    # seed, S, max_ctx, Hq, Hkv, d, dtype.  Contexts are cut into 1024-token
    # partitions on the VALU kernel (MHA) and on the matrix-core group
    # kernels (bf16 or fp32, two or more heads per KV head) for batches as
    # small as these (4096 tokens once the units fill a round of workgroups);
    # a longer context exercises the merge.
    (11, 7, 70, 4, 4, 64, "f32"),
    (12, 9, 1300, 2, 2, 128, "f32"),
    (13, 5, 4700, 8, 2, 128, "bf16"),
    (14, 12, 1100, 4, 4, 128, "bf16"),
    (15, 6, 1700, 4, 1, 64, "bf16"),
    (16, 10, 2100, 2, 2, 64, "f32"),
    (17, 3, 33, 16, 16, 128, "bf16"),
    (18, 9, 9000, 8, 2, 128, "f32"),       # fp32 group kernel, contexts split and merged
    (19, 11, 700, 12, 4, 64, "f32"),       # G = 3
]


@pytest.mark.parametrize("seed,S,max_ctx,hq,hkv,d,dtype", SMALL)
def test_small_ragged_batches(seed, S, max_ctx, hq, hkv, d, dtype):
    print(f"case: small seed={seed} S={S} ctx<={max_ctx} H={hq}/{hkv} d={d} {dtype}", flush=True)
    w = W.random_small(seed, S, max_ctx, hq, hkv, d, dtype)
    g, r = GpuReplay(w), _oracle(w)
    _check_state(g, r, w)
    err = _attn_err(g, r, w)
    assert err <= TOL[dtype], err


def test_13b_shaped_batch_full():
    w = W.shaped_13b()
    print(f"case: 13b S=64 ctx sum={sum(op[2] for op in w.ops if op[0]=='append')}", flush=True)
    g, r = GpuReplay(w), _oracle(w)
    _check_state(g, r, w)
    err = _attn_err(g, r, w)
    assert err <= TOL["bf16"], err


def test_13b_steps_in_the_bench_launch_configuration():
    """Three decode steps of the full 13B-shaped batch enqueued back to back the
    way bench.py times them: per step the batched slot reservation, the step's
    indices staged through a pinned buffer of its own and copied to the device
    in one packed copy on the launch stream (no host wait between steps), one
    pkv_decode_plan, then
    pkv_attention_decode_append (cache write, decode and the in-launch merge of
    split contexts) on two layers with pools of their own.  Every step's outputs
    of both layers against the oracle, and all four pools bit-exact at the end."""
    w = W.shaped_13b()
    print("case: 13b bench steps", flush=True)
    g, r = GpuReplay(w), _oracle(w)
    seqs = list(w.decode_seqs)
    S, H, D, steps = len(seqs), 40, 128, 3
    lens0 = np.array([r.alloc.num_tokens(s_) for s_ in seqs])
    assert lens0.max() > 1024              # some contexts split: the merge runs
    cap = int(lens0.max()) + steps
    MB = -(-cap // 16)
    # layer 1 has pools of its own (copies of layer 0's)
    gpools = [(g.k_pool, g.v_pool), (g.k_pool.clone(), g.v_pool.clone())]
    opools = [(r.k_pool, r.v_pool), (r.k_pool.copy(), r.v_pool.copy())]
    rng = np.random.default_rng(2024)

    def bf16(shape):
        return W.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))

    new = [[(bf16((S, H, D)), bf16((S, H, D)), bf16((S, H, D))) for _ in range(2)] for _ in range(steps)]
    dnew = [[tuple(rows_to_device(x, "cuda") for x in lay) for lay in st] for st in new]
    # packed staging: slots (int64), tables, lengths at 256-byte aligned offsets
    o_t = -(-S * 8 // 256) * 256
    o_l = o_t + -(-S * MB * 4 // 256) * 256
    nbytes = o_l + -(-S * 4 // 256) * 256

    def views(buf):
        return (buf[o_t:o_t + S * MB * 4].view(torch.int32).view(S, MB), buf[o_l:o_l + S * 4].view(torch.int32),
                buf[:S * 8].view(torch.int64))
    staging = [torch.zeros(nbytes, dtype=torch.uint8).pin_memory() for _ in range(steps)]
    buf_d = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    tables_d, lens_d, slots_d = views(buf_d)
    plan = torch.zeros(max(PK.pkv_decode_plan_bytes(S, cap), 256), dtype=torch.uint8, device="cuda")
    ws = PK.workspace_for(S, H, D, cap)
    outs = [[torch.full((S, H, D), -4.0, dtype=torch.float32, device="cuda") for _ in range(2)] for _ in range(steps)]
    host = []
    for k in range(steps):
        slots, cow = g.alloc.seq_append_slots_batch(seqs, [1] * S)
        assert len(cow) == 0
        t, ln = g.alloc.block_tables(seqs, MB)
        th, lh, sh = views(staging[k])
        sh.numpy()[:] = slots
        th.numpy()[:] = t
        lh.numpy()[:] = ln
        mcl = int(ln.max())
        buf_d.copy_(staging[k], non_blocking=True)
        PK.pkv_decode_plan(plan, lens_d, H, H, MB, mcl, PK.PKV_BF16)
        for lay in range(2):
            q, kn, vn = dnew[k][lay]
            PK.pkv_attention_decode_append(outs[k][lay], q, kn, vn, slots_d, gpools[lay][0], gpools[lay][1],
                                           tables_d, lens_d, mcl, float(w.scale), workspace=ws, plan=plan)
        host.append((list(slots), ln.copy()))
    torch.cuda.synchronize()
    for k in range(steps):
        oslots = []
        for s_ in seqs:
            sl, pairs = r.alloc.append_slots(s_, 1)
            oslots += sl
            assert not pairs
        assert host[k][0] == oslots
        otables = [r.alloc.block_table(s_) for s_ in seqs]
        olens = [r.alloc.num_tokens(s_) for s_ in seqs]
        assert list(host[k][1]) == olens
        for lay in range(2):
            q, kn, vn = new[k][lay]
            O.write_cache(opools[lay][0], opools[lay][1], kn, vn, oslots)
            ref = O.decode_attention(q, opools[lay][0], opools[lay][1], otables, olens, w.scale)
            err = float(np.abs(outs[k][lay].cpu().numpy() - ref).max())
            assert err <= TOL["bf16"], (k, lay, err)
    for (gk, gv), (ok, ov) in zip(gpools, opools):
        assert np.array_equal(pool_to_host(gk), ok) and np.array_equal(pool_to_host(gv), ov)


def test_gqa_batch_all_rows():
    print("case: gqa S=256 H=64/8, every row", flush=True)
    w, g, r = _big("gqa")
    _check_state(g, r, w)
    err = _attn_err(g, r, w)
    assert err <= TOL["bf16"], err


def test_parallel_sampling_all_rows():
    print("case: fork 32x8, every row", flush=True)
    w, g, r = _big("fork")
    _check_state(g, r, w)
    assert len(g.cow_pairs) == 32 * 7
    err = _attn_err(g, r, w)
    assert err <= TOL["bf16"], err


def test_long_context_decode_all_rows():
    print("case: long 16x32768 (+chunks), every decode row", flush=True)
    w, g, r = _big("long")
    _check_state(g, r, w)
    err = _attn_err(g, r, w)
    assert err <= TOL["bf16"], err


# ---------------------------------------------------------------------------
# Edge cases
# ---------------------------------------------------------------------------
def test_nan_in_unused_slots_never_reaches_the_output():
    w = W.random_small(21, 9, 90, 4, 2, 64, "bf16")
    print("case: nan poison", flush=True)
    g = GpuReplay(w, pool_fill=float("nan"))
    r = _oracle(w, pool_fill=np.uint16(0x7FC0))
    _check_state(g, r, w)
    err = _attn_err(g, r, w)
    assert err <= TOL["bf16"], err


def test_context_of_one_returns_the_value_row_and_zero_context_gives_zeros():
    w = W.random_small(22, 4, 1, 4, 4, 128, "f32")
    print("case: ctx 1 / 0", flush=True)
    g = GpuReplay(w)
    out, tables, lens = g.decode()
    for s in range(4):
        b = tables[s][0]
        v = g.v_pool[b, :, 0, :].cpu().numpy()
        assert np.array_equal(out[s], v)
    lens0 = np.array(lens).copy()
    lens0[1] = 0
    out0, _, _ = g.decode(tables=tables, lens=lens0, max_context_len=1)
    assert np.array_equal(out0[1], np.zeros_like(out0[1]))
    assert np.array_equal(out0[0], out[0])


@pytest.mark.parametrize("max_ctx", [150, 1500])
def test_physical_block_relabelling_gives_bit_identical_outputs(max_ctx):
    w = W.random_small(23, 6, max_ctx, 4, 4, 128, "bf16")
    print(f"case: relabel max_ctx={max_ctx}", flush=True)
    g = GpuReplay(w)
    out, tables, lens = g.decode()
    pi = torch.from_numpy(np.random.default_rng(0).permutation(w.num_blocks)).cuda()
    k2, v2 = torch.empty_like(g.k_pool), torch.empty_like(g.v_pool)
    k2[pi], v2[pi] = g.k_pool, g.v_pool
    g.k_pool, g.v_pool = k2, v2
    t2 = pi.cpu().numpy()[tables].astype(np.int32)
    out2, _, _ = g.decode(tables=t2, lens=lens)
    assert np.array_equal(out, out2)


def test_forked_samples_give_the_same_outputs_as_unshared_copies():
    w = W.parallel_sampling(seed=31, groups=2, samples=4, prompt=100, tail_hi=60, hq=4, d=128)
    print("case: fork vs unshared", flush=True)
    g = GpuReplay(w)
    out, tables, lens = g.decode()
    # unshared: each sample's full context written separately
    parent, rows_of, r, n = {}, {}, 0, 0
    for op in w.ops:
        if op[0] == "create":
            parent[n] = None; n += 1
        elif op[0] == "fork":
            parent[n] = op[1]; n += 1
        elif op[0] == "append":
            rows_of.setdefault(op[1], []).append((r, r + op[2])); r += op[2]
    ops, kr, vr = [], [], []
    for s in range(n):
        spans = ([] if parent[s] is None else rows_of[parent[s]][:1]) + rows_of[s]
        idx = np.concatenate([np.arange(a, b) for a, b in spans])
        ops += [("create",), ("append", s, len(idx)), ("flush",)]
        kr.append(w.k_rows[idx]); vr.append(w.v_rows[idx])
    w2 = W.Workload("unshared", w.dtype, w.num_heads, w.num_kv_heads, w.head_dim, 400,
                    np.arange(400, dtype=np.int32), ops, np.concatenate(kr), np.concatenate(vr),
                    w.decode_seqs, w.q, w.scale)
    g2 = GpuReplay(w2)
    out2, _, lens2 = g2.decode()
    assert list(lens) == list(lens2)
    assert np.array_equal(out, out2)


def test_bad_rows_are_nan_and_leave_other_rows_alone():
    w = W.random_small(24, 5, 1100, 2, 2, 64, "f32")
    print("case: bad rows", flush=True)
    g = GpuReplay(w)
    out, tables, lens = g.decode()
    t2 = np.array(tables).copy()
    l2 = np.array(lens).copy()
    t2[1, 0] = w.num_blocks + 5          # block id outside the pool
    t2[2, 0] = -3
    mcl = int(max(lens))
    l2[3] = mcl + 1                      # longer than max_context_len
    out2, _, _ = g.decode(tables=t2, lens=l2, max_context_len=mcl)
    assert np.isnan(out2[1]).all() and np.isnan(out2[2]).all() and np.isnan(out2[3]).all()
    # the other rows are computed exactly as before
    assert np.array_equal(out2[0], out[0]) and np.array_equal(out2[4], out[4])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_wide_groups_edges_and_bad_rows(dtype):
    """48 query heads over one KV head (17..64 per KV head: one workgroup for
    all three 16-row slices, K/V staged once in LDS): contexts of 1 and on
    and next to the 1024-token partition edges match the oracle; an empty
    context, an out-of-pool block id and a length past max_context_len give
    zero and NaN rows for those sequences only, the others keep their bits."""
    print(f"case: wide groups 48/1 edges and bad rows {dtype}", flush=True)
    w = W._plain_decode("wide", 91, [1, 1023, 1024, 1025, 2049, 17, 300, 3073], 48, 1, 128, dtype)
    g, r = GpuReplay(w), _oracle(w)
    err = _attn_err(g, r, w)
    assert err <= TOL[dtype], err
    out, tables, lens = g.decode()
    t2, l2 = np.array(tables).copy(), np.array(lens).copy()
    mcl = int(max(lens))
    l2[0] = 0
    t2[2, 0] = w.num_blocks + 3
    l2[5] = mcl + 1
    out2, _, _ = g.decode(tables=t2, lens=l2, max_context_len=mcl)
    assert (out2[0] == 0).all() and np.isnan(out2[2]).all() and np.isnan(out2[5]).all()
    for i in (1, 3, 4, 6, 7):
        assert np.array_equal(out2[i], out[i]), i


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_wide_groups_many_units_all_rows(dtype):
    """160 sequences of 200..2600 tokens, 64 query heads over 2 KV heads, d 64:
    about 300 units per KV head (1024-token partitions for float32, 2048 for
    bf16); for float32 that is two full rounds of one workgroup per CU and a
    partial third (the kernel deals every other round of 256 workgroups in
    reverse order).  Every output row against the oracle; the planned call
    gives the same bits."""
    print(f"case: wide groups many units 64/2 d=64 {dtype}", flush=True)
    w = W.random_small(97, 160, 2600, 64, 2, 64, dtype, min_ctx=200)
    g, r = GpuReplay(w), _oracle(w)
    out, tables, lens = g.decode()
    td, ld = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()
    mcl = int(lens.max())
    plan = PK.plan_for(ld, 64, 2, tables.shape[1], mcl, PK.PKV_BF16 if dtype == "bf16" else PK.PKV_F32)
    part = int(plan[16:20].view(torch.int32).item())
    assert part == (1024 if dtype == "f32" else 2048)        # three (two) workgroups per CU fill a round
    units = sum(-(-int(c) // part) for c in lens)
    if dtype == "f32":
        assert units * 2 > 2 * 256 and units * 2 % 256 != 0  # two full rounds and a partial one
    ref = O.decode_attention(w.q, r.k_pool, r.v_pool, [r.alloc.block_table(s) for s in w.decode_seqs],
                             [r.alloc.num_tokens(s) for s in w.decode_seqs], w.scale)
    err = float(np.abs(out - ref).max())
    assert err <= TOL[dtype], err
    out2 = torch.full((len(w.decode_seqs), 64, 64), -5.0, dtype=torch.float32, device="cuda")
    PK.pkv_attention_decode(out2, rows_to_device(w.q, "cuda"), g.k_pool, g.v_pool, td, ld, mcl, float(w.scale),
                            plan=plan)
    torch.cuda.synchronize()
    assert np.array_equal(out2.cpu().numpy(), out)


def test_append_skips_negative_and_out_of_pool_slots():
    w = W.random_small(25, 2, 20, 2, 2, 64, "bf16")
    print("case: append skips", flush=True)
    g = GpuReplay(w)
    before_k = pool_to_host(g.k_pool).copy()
    rows = rows_to_device(w.k_rows[:3], "cuda")
    sl = torch.tensor([-1, w.num_blocks * 16, w.num_blocks * 16 + 7], dtype=torch.int64, device="cuda")
    PK.pkv_append(g.k_pool, g.v_pool, rows, rows, sl)
    torch.cuda.synchronize()
    assert np.array_equal(pool_to_host(g.k_pool), before_k)


def test_workspace_reuse_across_calls_and_shapes():
    """One workspace (never cleared) serves consecutive calls with different batches."""
    print("case: workspace reuse", flush=True)
    ws = PK.workspace_for(16, 8, 128, 1600)
    results = []
    for seed, S, mx in ((41, 9, 1600), (42, 16, 700), (41, 9, 1600)):
        w = W.random_small(seed, S, mx, 8, 2, 128, "bf16")
        g = GpuReplay(w)
        tables, lens = g.tables(w.decode_seqs)
        out = torch.empty((S, 8, 128), dtype=torch.float32, device="cuda")
        PK.pkv_attention_decode(out, rows_to_device(w.q, "cuda"), g.k_pool, g.v_pool,
                                torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(),
                                int(lens.max()), float(w.scale), workspace=ws)
        torch.cuda.synchronize()
        r = _oracle(w)
        ref = O.decode_attention(w.q, r.k_pool, r.v_pool, [r.alloc.block_table(s) for s in w.decode_seqs],
                                 [r.alloc.num_tokens(s) for s in w.decode_seqs], w.scale)
        o = out.cpu().numpy()
        assert float(np.abs(o - ref).max()) <= TOL["bf16"]
        results.append(o)
    assert np.array_equal(results[0], results[2])


def test_planned_decode_matches_self_planned_and_reuses_the_plan():
    """One plan per step serves every layer: the planned call gives the same bits
    as the self-planning call, on two different pools with the same tables."""
    w = W.random_small(51, 11, 1400, 8, 8, 128, "bf16")
    print("case: planned decode", flush=True)
    g = GpuReplay(w)
    tables, lens = g.tables(w.decode_seqs)
    td, ld = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()
    mcl = int(lens.max())
    plan = PK.plan_for(ld, 8, 8, tables.shape[1], mcl, PK.PKV_BF16)
    q = rows_to_device(w.q, "cuda")
    pools = [(g.k_pool, g.v_pool), (g.v_pool, g.k_pool)]   # a second "layer": K and V swapped
    for kp, vp in pools:
        o1 = torch.empty((len(lens), 8, 128), dtype=torch.float32, device="cuda")
        o2 = torch.empty_like(o1)
        PK.pkv_attention_decode(o1, q, kp, vp, td, ld, mcl, float(w.scale))
        PK.pkv_attention_decode(o2, q, kp, vp, td, ld, mcl, float(w.scale), plan=plan)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)


def test_plan_built_for_other_sizes_gives_nan_rows():
    w = W.random_small(52, 4, 300, 2, 2, 64, "f32")
    print("case: plan mismatch", flush=True)
    g = GpuReplay(w)
    tables, lens = g.tables(w.decode_seqs)
    td, ld = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()
    mcl = int(lens.max())
    plan = PK.plan_for(ld, 2, 2, tables.shape[1], mcl + 1, PK.PKV_F32)   # built with another max_context_len
    o = torch.zeros((4, 2, 64), dtype=torch.float32, device="cuda")
    PK.pkv_attention_decode(o, rows_to_device(w.q, "cuda"), g.k_pool, g.v_pool, td, ld, mcl, float(w.scale),
                            plan=plan)
    torch.cuda.synchronize()
    assert torch.isnan(o).all()


_EDGES_4096 = [4095, 4096, 4097, 3, 8191, 8192, 8193, 700]


@pytest.mark.parametrize("ctxs,hq,hkv,dtype,part", [
    # the VALU kernel's 1024-token partitions (MHA)
    ([1023, 1024, 1025, 1, 16, 17, 2047, 2048, 2049, 3073], 4, 4, "bf16", 1024),
    # the matrix-core group kernels: few (sequence, KV head) pairs take
    # 1024-token partitions, so that the units fill a round of workgroups ...
    ([1023, 1024, 1025, 4095, 4096, 4097, 3, 2049], 8, 2, "bf16", 1024),
    ([1023, 1024, 1025, 4095, 4096, 4097, 3, 2049], 8, 2, "f32", 1024),
    # ... and 512 pairs over three 4096-token partitions already do
    (_EDGES_4096 * 8, 16, 8, "bf16", 4096),
    (_EDGES_4096 * 8, 16, 8, "f32", 4096),
])
def test_partition_boundaries(ctxs, hq, hkv, dtype, part):
    """Context lengths on and next to the partition edges of the decode kernels
    (the partition the library chose is read from the plan's header)."""
    print(f"case: partition edges {len(ctxs)} seqs H={hq}/{hkv} {dtype} part {part}", flush=True)
    w = W._plain_decode("edges", 77, ctxs, hq, hkv, 128, dtype)
    g, r = GpuReplay(w), _oracle(w)
    tables, lens = g.tables(w.decode_seqs)
    plan = PK.plan_for(torch.from_numpy(lens).cuda(), hq, hkv, tables.shape[1], int(lens.max()),
                       PK.PKV_BF16 if dtype == "bf16" else PK.PKV_F32)
    assert int(plan[16:20].view(torch.int32).item()) == part      # header word 4: tokens per partition
    err = _attn_err(g, r, w)
    assert err <= TOL[dtype], err


# ---------------------------------------------------------------------------
# Query-head groups (matrix-core decode kernels for bf16 and fp32 groups of
# two or more heads, in 16-row slices) and causal chunked prefill.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("seed,S,max_ctx,hq,hkv,d", [
    (71, 9, 1300, 16, 1, 128),    # G = 16: the whole MFMA row tile
    (72, 7, 600, 6, 2, 64),       # G = 3
    (73, 5, 900, 32, 1, 128),     # G = 32: two 16-row slices
    (74, 12, 40, 16, 8, 128),     # G = 2, short contexts (P rounding matters most)
    (75, 6, 2500, 64, 1, 128),    # G = 64: four slices
    (76, 5, 5000, 48, 2, 64),     # G = 24: slices of 16 and 8, contexts split past 4096
])
def test_query_head_groups(seed, S, max_ctx, hq, hkv, d, dtype):
    print(f"case: groups seed={seed} H={hq}/{hkv} d={d} {dtype}", flush=True)
    w = W.random_small(seed, S, max_ctx, hq, hkv, d, dtype)
    g, r = GpuReplay(w), _oracle(w)
    err = _attn_err(g, r, w)
    assert err <= TOL[dtype], err


def _prefill_ref(r, w, rows=None):
    tables = [r.alloc.block_table(s) for s in w.chunk_seqs]
    lens = [r.alloc.num_tokens(s) for s in w.chunk_seqs]
    return O.prefill_chunk_attention(w.chunk_q, w.chunk_query_start_loc, r.k_pool, r.v_pool, tables, lens, w.scale)


PREFILL = [
    # seed, contexts, chunk lengths, Hq, Hkv, d
    (61, [60, 300, 700], [37, 64, 100], 8, 2, 128),
    (62, [16, 33, 129, 1], [16, 1, 129, 1], 4, 4, 64),      # whole prompt, single query, MHA
    (63, [1000], [200], 16, 2, 128),
    (64, [90, 45], [90, 5], 32, 1, 128),                    # MQA: 32 heads per KV head
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("seed,ctxs,nqs,hq,hkv,d", PREFILL)
def test_prefill_chunks(seed, ctxs, nqs, hq, hkv, d, dtype):
    """bf16 pools on the bf16 matrix-core kernel, float32 pools on the fp32
    one; every query row against the oracle."""
    print(f"case: prefill {dtype} seed={seed} ctx={ctxs} n={nqs} H={hq}/{hkv} d={d}", flush=True)
    w = W.random_prefill(seed, ctxs, nqs, hq, hkv, d, dtype=dtype)
    g, r = GpuReplay(w), _oracle(w)
    out, _, _ = g.prefill()
    ref = _prefill_ref(r, w)
    assert np.isfinite(out).all()
    err = float(np.abs(out - ref).max())
    assert err <= TOL[dtype], err


def test_prefill_f32_long_chunks():
    """float32 chunks over a few thousand keys (rounding accumulated over
    hundreds of 16-key tiles stays within 1e-5), 64 and 128 dims."""
    for seed, ctxs, nqs, hq, hkv, d in [(71, [4700, 1500], [300, 1500], 8, 2, 128), (72, [3000], [700], 4, 4, 64)]:
        print(f"case: prefill f32 long seed={seed} ctx={ctxs} n={nqs}", flush=True)
        w = W.random_prefill(seed, ctxs, nqs, hq, hkv, d, dtype="f32")
        g, r = GpuReplay(w), _oracle(w)
        out, _, _ = g.prefill()
        assert np.isfinite(out).all()
        err = float(np.abs(out - _prefill_ref(r, w)).max())
        assert err <= TOL["f32"], err


def _bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _raises(scores_log2, threshold=8.0, step=32):
    """How often a running maximum kept within `threshold` of the scores seen
    so far is raised, keys taken `step` at a time (scores in log2 units)."""
    top, n = -np.inf, 0
    for j in range(0, len(scores_log2), step):
        m = float(np.max(scores_log2[j:j + step]))
        if m > top + threshold:
            top, n = m, n + 1
    return n


def test_prefill_rows_whose_maximum_rises_through_the_keys():
    """Keys that rise along the context (each row's running maximum is raised
    and its accumulators rescaled again and again) and scores spread over
    hundreds of log2 units, so early keys' probabilities underflow."""
    ctxs, nqs = [900, 333], [300, 77]
    w = W.random_prefill(67, ctxs, nqs, 8, 2, 128)
    rng = np.random.default_rng(67)
    q = np.abs(rng.standard_normal((int(sum(nqs)), 8, 128), dtype=np.float32))
    w.chunk_q = W.f32_to_bf16_bits(q)
    pos = np.concatenate([np.arange(c) for c in ctxs]).astype(np.float32)
    w.k_rows = W.f32_to_bf16_bits(0.5 * _bf16_to_f32(w.k_rows) + (0.02 * pos)[:, None, None])
    print("case: prefill rising maxima", flush=True)
    g, r = GpuReplay(w), _oracle(w)
    # the last query of sequence 0, head 0 (KV head 0): its running maximum is
    # raised many times
    k0 = _bf16_to_f32(w.k_rows[:ctxs[0], 0]).astype(np.float64)
    s_log2 = k0 @ _bf16_to_f32(w.chunk_q[nqs[0] - 1, 0]).astype(np.float64) * float(w.scale) / np.log(2)
    assert _raises(s_log2) >= 20
    out, _, _ = g.prefill()
    assert np.isfinite(out).all()
    err = float(np.abs(out - _prefill_ref(r, w)).max())
    assert err <= TOL["bf16"], err


def test_prefill_with_a_wide_score_range():
    """Scale 1 on random rows: scores of standard deviation ~11 (16 log2 units)."""
    w = W.random_prefill(68, [700, 150, 40], [120, 150, 7], 16, 4, 128)
    w.scale = np.float32(1.0)
    print("case: prefill wide scores", flush=True)
    g, r = GpuReplay(w), _oracle(w)
    out, _, _ = g.prefill()
    assert np.isfinite(out).all()
    err = float(np.abs(out - _prefill_ref(r, w)).max())
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("scale,dtype", [(-0.3, "bf16"), (0.0, "bf16"), (-1.0, "bf16"),
                                         (-0.3, "f32"), (0.0, "f32"), (-0.0884, "f32")])
def test_prefill_with_negative_and_zero_scales(scale, dtype):
    """Any finite scale, as decode takes: a negative one reverses the scores'
    order, zero weighs every visible key the same.  float32 takes scales of
    the size attention uses (up to a few times 1/sqrt(d)): at |scale| = 1 with
    128 dims the scores reach +-40, and rounding them to float32 alone moves
    outputs by about 1e-5, the float32 bar itself."""
    w = W.random_prefill(69, [500, 90, 33], [70, 90, 3], 8, 2, 128, dtype=dtype)
    w.scale = np.float32(scale)
    print(f"case: prefill {dtype} scale {scale}", flush=True)
    g, r = GpuReplay(w), _oracle(w)
    out, _, _ = g.prefill()
    assert np.isfinite(out).all()
    err = float(np.abs(out - _prefill_ref(r, w)).max())
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_nan_in_unused_slots_never_reaches_the_output(dtype):
    w = W.random_prefill(65, [70, 33], [20, 33], 8, 2, 128, dtype=dtype)
    print(f"case: prefill {dtype} nan poison", flush=True)
    g = GpuReplay(w, pool_fill=float("nan"))
    r = _oracle(w, pool_fill=np.uint16(0x7FC0) if dtype == "bf16" else np.float32("nan"))
    out, _, _ = g.prefill()
    err = float(np.abs(out - _prefill_ref(r, w)).max())
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_block_id_outside_the_pool_gives_nan_rows(dtype):
    """A table entry outside [0, num_blocks) in a sequence's first block: every
    row of that sequence is NaN (every row's keys start there); the other
    sequences come out as without it."""
    w = W.random_prefill(70, [300, 120, 64], [100, 20, 64], 8, 2, 128, dtype=dtype)
    print(f"case: prefill {dtype} bad block id", flush=True)
    g = GpuReplay(w)
    out, tables, lens = g.prefill()
    t2 = np.array(tables).copy()
    t2[1, 0] = w.num_blocks + 3
    out2, _, _ = g.prefill(tables=t2, lens=lens)
    qsl = w.chunk_query_start_loc
    assert np.isnan(out2[qsl[1]:qsl[2]]).all()
    assert np.array_equal(out2[:qsl[1]], out[:qsl[1]]) and np.array_equal(out2[qsl[2]:], out[qsl[2]:])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_bad_rows(dtype):
    """A chunk longer than its context gets NaN rows; a query range outside the
    query buffer is not written; other sequences are computed as before."""
    w = W.random_prefill(66, [50, 80, 64], [10, 20, 30], 8, 2, 128, dtype=dtype)
    print(f"case: prefill {dtype} bad rows", flush=True)
    g = GpuReplay(w)
    out, tables, lens = g.prefill()
    l2 = np.array(lens).copy()
    l2[0] = 5                                   # context shorter than the 10-query chunk
    out2, _, _ = g.prefill(tables=tables, lens=l2, max_context_len=int(max(lens)))
    qsl = w.chunk_query_start_loc
    assert np.isnan(out2[qsl[0]:qsl[1]]).all()
    assert np.array_equal(out2[qsl[1]:], out[qsl[1]:])
    qsl3 = qsl.copy()
    qsl3[3] = qsl3[3] + 5                       # last range runs past the buffer: skipped
    out3, _, _ = g.prefill(qsl=qsl3, tables=tables, lens=lens, max_query_len=35)
    assert (out3[qsl[2]:] == -7.0).all()
    assert np.array_equal(out3[:qsl[2]], out[:qsl[2]])


def test_long_context_prefill_all_queries():
    print("case: long mix prefill 4x512 on 8192, every query row", flush=True)
    w, g, r = _big("long")
    out, _, _ = g.prefill()
    assert np.isfinite(out).all()
    ref = _prefill_ref(r, w)
    assert out.shape == ref.shape == (4 * 512, 32, 128)
    err = float(np.abs(out - ref).max())
    assert err <= TOL["bf16"], err
    _BIG.clear()
