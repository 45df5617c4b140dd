"""Decode with the step's cache write (pkv_attention_decode_append) against the
oracle's two steps -- write each sequence's new token at its slot, then decode
over the whole context: pools bit-exact afterwards, outputs within 1e-5 (fp32)
/ 2e-3 (bf16), on the VALU kernel (MHA, fp32) and the MFMA group kernel
(GQA), at block sizes 8, 16 and 32, across partition splits, with sequences that have no
new token (slot -1), a slot that is not the last token's (NaN rows, nothing
written) and a planned call."""
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


def _rows(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    return x if dtype == "f32" else W.f32_to_bf16_bits(x)


def _run(w, seed, no_new=(), wrong=(), planned=False):
    g = GpuReplay(w)
    r = O.replay(w.ops, w.k_rows, w.v_rows, w.num_blocks, w.num_kv_heads, w.head_dim, w.initial_free_order,
                 block_size=w.block_size)
    seqs = list(w.decode_seqs)
    S = len(seqs)
    bs = w.block_size
    slots = np.full(S, -1, dtype=np.int64)
    for i, s in enumerate(seqs):
        if i in no_new:
            continue
        sl, pairs = g.alloc.seq_append_slots(s, 1)
        osl, opairs = r.alloc.append_slots(s, 1)
        assert list(sl) == osl and [tuple(p) for p in pairs] == opairs
        assert not pairs          # fresh tails: no copy-on-write in these workloads
        slots[i] = sl[0]
    rng = np.random.default_rng(seed)
    kn = _rows(rng, (S, w.num_kv_heads, w.head_dim), w.dtype)
    vn = _rows(rng, (S, w.num_kv_heads, w.head_dim), w.dtype)
    tables, lens = g.tables(seqs)
    dslots = slots.copy()
    for i in wrong:
        # a slot inside the sequence's table that is not its last token's
        dslots[i] = int(tables[i, 0]) * bs
    write = [i for i in range(S) if slots[i] >= 0 and i not in wrong]
    O.write_cache(r.k_pool, r.v_pool, kn[write], vn[write], slots[write], bs)
    td, ld = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()
    mcl = int(lens.max())
    plan = None
    if planned:
        plan = PK.plan_for(ld, w.num_heads, w.num_kv_heads, tables.shape[1], mcl,
                           PK.PKV_BF16 if w.dtype == "bf16" else PK.PKV_F32, block_size=bs)
    out = torch.full((S, w.num_heads, w.head_dim), -2.0, dtype=torch.float32, device="cuda")
    PK.pkv_attention_decode_append(out, rows_to_device(w.q, "cuda"), rows_to_device(kn, "cuda"),
                                   rows_to_device(vn, "cuda"), torch.from_numpy(dslots).cuda(), g.k_pool, g.v_pool,
                                   td, ld, mcl, float(w.scale), plan=plan)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.array_equal(pool_to_host(g.k_pool), r.k_pool) and np.array_equal(pool_to_host(g.v_pool), r.v_pool)
    ok = [i for i in range(S) if i not in wrong]
    ref = O.decode_attention(w.q[ok], r.k_pool, r.v_pool, [r.alloc.block_table(seqs[i]) for i in ok],
                             [r.alloc.num_tokens(seqs[i]) for i in ok], w.scale, block_size=bs)
    err = float(np.abs(o[ok] - ref).max())
    assert err <= TOL[w.dtype], err
    for i in wrong:
        assert np.isnan(o[i]).all()
    return err


@pytest.mark.parametrize("seed,S,max_ctx,hq,hkv,d,dtype,bs", [
    (1, 7, 300, 4, 4, 64, "f32", 16),
    (2, 9, 2500, 8, 8, 128, "bf16", 16),     # split contexts on the VALU kernel
    (3, 6, 5000, 16, 2, 128, "bf16", 16),    # MFMA group kernel, split contexts
    (4, 5, 900, 8, 2, 64, "f32", 16),        # fp32 group kernel
    (5, 7, 700, 4, 4, 128, "bf16", 8),
    (6, 7, 1300, 8, 8, 64, "f32", 32),
    (7, 6, 5000, 16, 2, 128, "bf16", 8),     # MFMA group kernel: two 8-token blocks per 16-key tile
    (8, 6, 5000, 16, 2, 128, "bf16", 32),    # MFMA group kernel: two 16-key tiles per block
    (9, 9, 300, 8, 4, 64, "bf16", 8),        # the new token in either half of a tile
    (10, 6, 5000, 8, 2, 128, "f32", 8),      # fp32 group kernel, split contexts, 8-token blocks
    (11, 7, 400, 16, 4, 128, "f32", 32),     # fp32 group kernel, 32-token blocks
    (12, 5, 4500, 32, 1, 128, "bf16", 16),   # two 16-row slices (the first one stores the row)
    (13, 4, 900, 64, 2, 64, "f32", 8),       # fp32, two slices
    (14, 5, 3000, 64, 1, 128, "bf16", 8),    # wide group kernel (four slices in one workgroup), split contexts
    (15, 6, 700, 24, 1, 64, "bf16", 32),     # wide group kernel, 32-token blocks
    (16, 5, 3000, 64, 1, 128, "f32", 16),    # float32 wide group kernel, split contexts
    (17, 6, 700, 32, 1, 64, "f32", 8),       # float32 wide group kernel, 8-token blocks
])
def test_decode_append_matches_write_then_decode(seed, S, max_ctx, hq, hkv, d, dtype, bs):
    print(f"case: decode_append seed={seed} {dtype} {hq}/{hkv} d={d} bs={bs}", flush=True)
    w = W.random_small(seed + 300, S, max_ctx, hq, hkv, d, dtype, block_size=bs)
    _run(w, seed)
    _run(w, seed + 1, planned=True)


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_no_new_token_and_a_wrong_slot(bs):
    print(f"case: decode_append -1 and wrong slots bs={bs}", flush=True)
    for hq, hkv, dtype in ((8, 8, "bf16"), (16, 2, "bf16"), (16, 2, "f32"), (32, 1, "bf16"), (32, 1, "f32")):
        w = W.random_small(77, 8, 700, hq, hkv, 128, dtype, block_size=bs)
        _run(w, 9, no_new=(1, 4), wrong=(2, 6))


def test_13b_batch_with_the_cache_write():
    print("case: decode_append 13b", flush=True)
    w = W.shaped_13b()
    _run(w, 11, planned=True)
