"""Benchmark: one decode step of the 13B-shaped batch through libpkv on one GPU.

A step is one pass of the hot path over the batch: the host allocator reserves
one new slot per sequence (and names any copy-on-write pairs), the slot map,
block tables and context lengths go to the device in one packed copy and the
decode plan is built from them, and then for each of the 40 layers one call writes the new
token's K/V into that layer's paged pool and runs paged decode attention over
it (pkv_attention_decode_append: the cache write and the merge of split
contexts happen inside the decode launch).

Workload: 64 sequences, 40 MHA heads, head_dim 128, bf16, context lengths
lognormal (median 200, sigma 1.0) clipped to [1, 2048], 16-token blocks shuffled
over a pool of 1.2x the blocks needed, one pool per layer (40 pools, ~21 GB, far
larger than the 256 MB last-level cache).  Pool contents, queries and new K/V
are synthetic N(0, 1) bf16 drawn on the device; the inputs are resident in HBM
before the timed region starts.

Prints one JSON line: decode tokens/s (value), effective KV GB/s and the
fraction of the 8 TB/s HBM peak, a roofline object for the decode kernel, and
the CPU oracle's rate on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
FP32_MFMA_PEAK_TFLOPS = 157.3   # dense fp32 matrix-core peak of the MI355X
METRIC = "paged decode attention: KV GB/s and % of HBM peak; decode tokens/s per step"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_13b_counters.md")
# the sources the headline decode kernel is built from
KERNEL_SRCS = [os.path.join(ROOT, "paged_kv_cache_171_amd", "csrc", f)
               for f in ("pkv_kernels.hip", "pkv_decode_valu.h", "pkv_device.h", "pkv_internal.h")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(alg_bytes_per_launch: float):
    """HBM bytes per decode launch from the committed counter summary, if it was
    taken on the current kernel source (else None).  The summary holds the
    counter bytes of its own run and that run's algorithmic bytes; the traffic
    is scaled by the ratio of algorithmic bytes to this run's launches."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    text = open(COUNTERS_FILE).read()
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    a = re.search(r"alg_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not h or not t or not a or h.group(1) != kernel_source_hash():
        return None
    return round(float(t.group(1)) * alg_bytes_per_launch / float(a.group(1)))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=40)
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time for the oracle sample")
    ap.add_argument("--workload", default="13b",
                    choices=["13b", "gqa", "fork", "long", "swap", "serve", "blocksize", "probes"],
                    help="13b: the headline decode step (default).  gqa / fork / long: kernel measurements on the "
                         "grouped-query, parallel-sampling and long-context + chunked-prefill batches.  swap: "
                         "block copies between HBM and pinned host memory.  serve: the continuous-batching loop "
                         "(continuous vs static policy) over a request stream.  blocksize: the 13B-shaped decode "
                         "with 8-, 16- and 32-token blocks.  probes: streaming-read and decode-access-pattern "
                         "read ceilings")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run pkv_copy_blocks over 4096 whole blocks (a plain copy of known size, "
                         "used to scale the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def copy_probe():
    """Copy 4096 whole 40-head bf16 blocks of K and of V (2 x 640 MiB read,
    2 x 640 MiB written) three times with pkv_copy_blocks."""
    import torch
    import paged_kv_cache_171_amd as PK
    dev = torch.device("cuda:0")
    n, H, D, P = 4096, 40, 128, 16
    k = torch.zeros(2 * n, H, P, D, dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    pairs = torch.stack([torch.arange(n), torch.arange(n, 2 * n)], 1).to(torch.int32).to(dev)
    for _ in range(3):
        PK.pkv_copy_blocks(k, v, pairs)
    torch.cuda.synchronize()
    block_bytes = H * P * D * 2
    print(json.dumps({"copy_probe": "pkv_copy_blocks", "pairs": n, "read_bytes": 2 * n * block_bytes,
                      "write_bytes": 2 * n * block_bytes, "launches": 3}), flush=True)


def _host_bits(t):
    """A device tensor's storage as numpy (bf16 as its uint16 bits)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def cpu_baseline(layers, tables, lens, scale, target_s: float, tol: float):
    """The oracle (float64 numpy) on the inputs of the last timed step, as the
    GPU saw them: for layers taken in turn (first, last, second, ...), that
    layer's pools, queries and outputs are copied to the host, the oracle
    decodes all 64 sequences three times on one BLAS thread (best of 3), and
    its outputs are compared with the GPU's; until ~target_s seconds of oracle
    time.  Then one layer again with the BLAS threads at their default (all
    host cores).  layers(l) -> (q, k_pool, v_pool, out) device tensors."""
    from threadpoolctl import threadpool_limits
    from oracle import pkv_oracle as O

    n_layers = layers(None)
    order = []
    lo, hi = 0, n_layers - 1
    while lo <= hi:
        order.append(lo)
        if hi != lo:
            order.append(hi)
        lo, hi = lo + 1, hi - 1
    best, spent, err, rows, done = [], 0.0, 0.0, 0, 0
    first = None
    for l in order:
        q, kp, vp, out = (_host_bits(x) if i < 3 else x.cpu().numpy() for i, x in enumerate(layers(l)))
        if first is None:
            first = (q, kp, vp)
        ts = []
        with threadpool_limits(limits=1):
            for _ in range(3):
                t0 = time.perf_counter()
                ref = O.decode_attention(q, kp, vp, tables, lens, scale)
                ts.append(time.perf_counter() - t0)
        spent += sum(ts)
        best.append(min(ts))
        err = max(err, float(np.abs(out - ref).max()))
        rows += out.shape[0] * out.shape[1]
        done += 1
        if spent >= target_s:
            break
    per_layer = float(np.median(best))
    tok_s = len(lens) / (per_layer * n_layers)
    cores = os.cpu_count() or 1
    q, kp, vp = first
    ts = []
    for _ in range(3):
        t0 = time.perf_counter()
        O.decode_attention(q, kp, vp, tables, lens, scale)
        ts.append(time.perf_counter() - t0)
    tok_s_all = len(lens) / (min(ts) * n_layers)
    return {"value": round(tok_s, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of the {n_layers} layers of the last timed step (64 seqs, {int(np.sum(lens))} "
                      f"cached tokens, the GPU's own pools and queries, 40 heads x 128, bf16 inputs, float64 "
                      f"math), each best of 3 on one thread ({spent:.1f} s in all); median layer time scaled "
                      f"to a {n_layers}-layer step",
            "max_abs_err": err, "tol": tol, "rows_checked": rows,
            "all_cores": {"value": round(tok_s_all, 3), "cores": cores,
                          "sample": "the first sampled layer, best of 3, BLAS threads at their default"}}


def secondary_cpu_check(name, cases, target_s: float):
    """The oracle on a few rows of a secondary workload's last call (its own
    inputs, copied from the device): max abs error and the oracle's rate.
    cases: list of (label, fn) where fn() -> (oracle output, GPU output, rows)."""
    from threadpoolctl import threadpool_limits
    res = {"kind": "oracle", "cores": 1}
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        for label, fn in cases:
            t1 = time.perf_counter()
            ref, got, rows = fn()
            dt = time.perf_counter() - t1
            res[f"{label}_max_abs_err"] = float(np.abs(got - ref).max())
            res[f"{label}_rows_checked"] = rows
            res[f"{label}_oracle_rows_per_s"] = round(rows / dt, 2)
            if time.perf_counter() - t0 > target_s:
                break
    res["tol"] = 2e-3
    if any(label.endswith("_f32") for label, _ in cases):
        res["f32_tol"] = 1e-5
    res["seconds"] = round(time.perf_counter() - t0, 1)
    return res


def _timed(fn, reps, stream):
    """Average duration (us) of fn() over reps calls, HIP events on `stream`."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / reps * 1e3


def tile_read_ceiling(pools, tables_h, lens_h, num_kv_heads, stream, reps) -> dict:
    """The read-only probe of a batch's own access pattern (tile_read_kernel:
    whole 4 KiB K and V tiles through the tables, one workgroup per (16-block
    chunk, KV head), full chunks first, nothing computed), timed over the same
    bf16 layer pools as the decode it bounds."""
    import torch
    P = 16
    dev = pools[0][0].device
    nblk = -(-lens_h // P)
    work = [(s_, c) for s_ in range(len(lens_h)) for c in range(-(-int(nblk[s_]) // 16))]
    work.sort(key=lambda sc: -min(16, int(nblk[sc[0]]) - 16 * sc[1]))
    work_d = torch.tensor(work, dtype=torch.int32, device=dev)
    td, ld = torch.from_numpy(np.ascontiguousarray(tables_h)).to(dev), torch.from_numpy(lens_h).to(dev)
    sink = torch.zeros(len(work) * num_kv_heads * 4, dtype=torch.int32, device=dev)
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_171_amd", "libpkv_probes.so"))
    lib.pkvprobe_tile_read.restype = ctypes.c_int
    sp = stream.cuda_stream

    def all_layers():
        for kp, vp in pools:
            rc = lib.pkvprobe_tile_read(ctypes.c_void_p(kp.data_ptr()), ctypes.c_void_p(vp.data_ptr()),
                                        ctypes.c_void_p(td.data_ptr()), int(tables_h.shape[1]),
                                        ctypes.c_void_p(ld.data_ptr()), P, ctypes.c_void_p(work_d.data_ptr()),
                                        len(work), num_kv_heads, 4096, ctypes.c_void_p(sink.data_ptr()),
                                        ctypes.c_void_p(sp))
            if rc != 0:
                raise RuntimeError(f"tile_read launch failed: {rc}")
    us = _median_us(all_layers, stream, reps) / len(pools)
    kv = int(lens_h.sum()) * 2 * num_kv_heads * 128 * 2
    return {"us_per_layer": round(us, 2), "gbps": round(kv / us / 1e3, 1),
            "hbm_peak_frac": round(kv / us / 1e3 / HBM_PEAK_GBPS, 4)}


def secondary(args):
    """Kernel measurements on the other batches (one JSON line each; not the headline).

    gqa:  256 seqs, 64 query / 8 KV heads, d 128, bf16, ctx U[128, 4096], pool 1.2x
          shuffled, 8 layer pools: decode (MFMA group kernel) per layer; then 2
          float32 layers, and 2 layers of one KV head for the 64 query heads (the
          wide group kernel) and for 16 of them.
    fork: 32 groups x 8 samples of a 1000-token prompt, tails U[1, 512], 40 heads x
          128 (13B-shaped), 40 layer pools like the headline's: the copy-on-write
          copies, then decode over the shared blocks (the shared-prefix plan built
          once per step, for all 40 layers); then plain and shared-prefix decode
          over 2 float32 layers of the same tables.
    long: 16 seqs at ctx 32768 (8 partitions of 4096 each) + 4 prefill chunks of
          512 causal queries ending 8192-token contexts, 32 / 8 heads, 4 layer pools.
    """
    import torch
    import paged_kv_cache_171_amd as PK
    import pkv_workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    P, D = 16, 128
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)

    name = args.workload
    w = {"gqa": lambda: W.gqa(with_rows=False), "fork": lambda: W.parallel_sampling(with_rows=False),
         "long": lambda: W.long_mix(with_rows=False)}[name]()
    L = {"gqa": 8, "fork": 40, "long": 4}[name]
    Hq, Hkv, NB = w.num_heads, w.num_kv_heads, w.num_blocks
    alloc = PK.BlockAllocator(NB, P, w.initial_free_order)
    pairs = []
    for op in w.ops:                      # the allocator script: tables, slots and copy pairs
        if op[0] == "create":
            alloc.seq_create()
        elif op[0] == "fork":
            alloc.seq_fork(op[1])
        elif op[0] == "append":
            pairs += alloc.seq_append_slots(op[1], op[2])[1]
    seqs = w.decode_seqs
    lens_h = np.array([alloc.seq_block_table(s)[1] for s in seqs], dtype=np.int32)
    MB = int(-(-lens_h.max() // P))
    tables_h, _ = alloc.block_tables(seqs, MB)
    pools = [(randn(NB, Hkv, P, D), randn(NB, Hkv, P, D)) for _ in range(L)]
    q = randn(len(seqs), Hq, D)
    out = torch.empty(len(seqs), Hq, D, dtype=torch.float32, device=dev)
    td, ld = torch.from_numpy(tables_h).to(dev), torch.from_numpy(lens_h).to(dev)
    mcl = int(lens_h.max())
    ws = PK.workspace_for(len(seqs), Hq, D, mcl, device=dev)
    plan = PK.plan_for(ld, Hq, Hkv, MB, mcl, PK.PKV_BF16)
    scale = 1.0 / math.sqrt(D)
    reps = max(args.steps, 3)

    def decode_all():
        for kp, vp in pools:
            PK.pkv_attention_decode(out, q, kp, vp, td, ld, mcl, scale, workspace=ws, plan=plan)

    for _ in range(max(args.warmup, 1)):
        decode_all()
    torch.cuda.synchronize()
    dec_us = _timed(decode_all, reps, stream) / L
    kv_logical = int(lens_h.sum()) * 2 * Hkv * D * 2
    res = {"workload": name, "layers": L, "num_seqs": len(seqs), "heads": f"{Hq}/{Hkv}", "head_dim": D,
           "mean_ctx": round(float(lens_h.mean()), 1), "decode_us_per_layer": round(dec_us, 2),
           "decode_kv_gbps": round(kv_logical / dec_us / 1e3, 1),
           "decode_hbm_peak_frac": round(kv_logical / dec_us / 1e3 / HBM_PEAK_GBPS, 4),
           "decode_tokens_per_s_per_layer": round(len(seqs) / dec_us * 1e6, 1),
           "kernel": "decode_group_mfma_kernel" if 2 <= Hq // Hkv <= 16 else "decode_valu_kernel"}
    if name in ("gqa", "long"):
        # the same tables read with nothing computed: the ceiling of this access pattern
        tr = tile_read_ceiling(pools, tables_h, lens_h, Hkv, stream, reps)
        res.update({"tile_read_us_per_layer": tr["us_per_layer"], "tile_read_gbps": tr["gbps"],
                    "decode_frac_of_tile_read": round(tr["us_per_layer"] / dec_us, 4)})
    if name == "gqa":
        # the same batch over float32 pools (2 layers of the same tables): the
        # fp32 matrix-core group kernel, against HBM peak like the bf16 line
        fpools = [(torch.randn(NB, Hkv, P, D, generator=gen, device=dev),
                   torch.randn(NB, Hkv, P, D, generator=gen, device=dev)) for _ in range(2)]
        q32 = torch.randn(len(seqs), Hq, D, generator=gen, device=dev)
        out32 = torch.empty_like(out)
        plan32 = PK.plan_for(ld, Hq, Hkv, MB, mcl, PK.PKV_F32)

        def decode_f32_all():
            for kp, vp in fpools:
                PK.pkv_attention_decode(out32, q32, kp, vp, td, ld, mcl, scale, workspace=ws, plan=plan32)
        decode_f32_all()
        torch.cuda.synchronize()
        d32_us = _timed(decode_f32_all, reps, stream) / len(fpools)
        kv32 = kv_logical * 2
        res.update({"decode_f32_us_per_layer": round(d32_us, 2), "decode_f32_kv_gbps": round(kv32 / d32_us / 1e3, 1),
                    "decode_f32_hbm_peak_frac": round(kv32 / d32_us / 1e3 / HBM_PEAK_GBPS, 4),
                    "decode_f32_kernel": "decode_group_f32_kernel"})
        # one KV head for all 64 query heads (the same tables, a pool of one
        # head, 2 layers): the group kernel in four 16-row slices
        mpools = [(randn(NB, 1, P, D), randn(NB, 1, P, D)) for _ in range(2)]
        mplan = PK.plan_for(ld, Hq, 1, MB, mcl, PK.PKV_BF16)

        def decode_mqa_all():
            for kp, vp in mpools:
                PK.pkv_attention_decode(out, q, kp, vp, td, ld, mcl, scale, workspace=ws, plan=mplan)
        decode_mqa_all()
        torch.cuda.synchronize()
        mq_us = _timed(decode_mqa_all, reps, stream) / len(mpools)
        res.update({"decode_64x1_us_per_layer": round(mq_us, 2),
                    "decode_64x1_kv_gbps": round(kv_logical / Hkv / mq_us / 1e3, 1)})
        # the same tables over the one-head pools read with nothing computed
        # (4 KiB K and V tiles, one per block: the ceiling of this access pattern)
        tr1 = tile_read_ceiling(mpools, tables_h, lens_h, 1, stream, reps)
        res.update({"decode_64x1_tile_read_us_per_layer": tr1["us_per_layer"],
                    "decode_64x1_tile_read_gbps": tr1["gbps"],
                    "decode_64x1_frac_of_tile_read": round(tr1["us_per_layer"] / mq_us, 4)})
        # the same over float32 pools of the one head: the float32 wide group kernel
        mpools32 = [(torch.randn(NB, 1, P, D, generator=gen, device=dev),
                     torch.randn(NB, 1, P, D, generator=gen, device=dev)) for _ in range(2)]
        mplan32 = PK.plan_for(ld, Hq, 1, MB, mcl, PK.PKV_F32)

        def decode_mqa_f32_all():
            for kp, vp in mpools32:
                PK.pkv_attention_decode(out32, q32, kp, vp, td, ld, mcl, scale, workspace=ws, plan=mplan32)
        decode_mqa_f32_all()
        torch.cuda.synchronize()
        mq32_us = _timed(decode_mqa_f32_all, reps, stream) / len(mpools32)
        res.update({"decode_64x1_f32_us_per_layer": round(mq32_us, 2),
                    "decode_64x1_f32_kv_gbps": round(kv_logical * 2 / Hkv / mq32_us / 1e3, 1),
                    "decode_64x1_f32_mfma_tflops": round(4 * Hq * D * int(lens_h.sum()) / mq32_us / 1e6, 1),
                    "decode_64x1_f32_partition_tokens": int(mplan32[16:20].view(torch.int32).item())})
        del mpools32
        # 16 query heads over the one KV head: 256 (sequence, KV head) pairs,
        # so the library cuts contexts into 1024-token partitions to fill the CUs
        q16 = q[:, :16].contiguous()
        out16 = torch.empty(len(seqs), 16, D, dtype=torch.float32, device=dev)
        plan16 = PK.plan_for(ld, 16, 1, MB, mcl, PK.PKV_BF16)

        def decode_16x1_all():
            for kp, vp in mpools:
                PK.pkv_attention_decode(out16, q16, kp, vp, td, ld, mcl, scale, workspace=ws, plan=plan16)
        decode_16x1_all()
        torch.cuda.synchronize()
        m16_us = _timed(decode_16x1_all, reps, stream) / len(mpools)
        res.update({"decode_16x1_us_per_layer": round(m16_us, 2),
                    "decode_16x1_kv_gbps": round(kv_logical / Hkv / m16_us / 1e3, 1),
                    "decode_16x1_partition_tokens": int(plan16[16:20].view(torch.int32).item())})
        del mpools
    if name == "fork":
        unique = len({int(b) for s, c in zip(range(len(seqs)), lens_h) for b in tables_h[s, :-(-int(c) // P)]})
        res["kv_unique_bytes"] = unique * P * 2 * Hkv * D * 2
        res["kv_logical_bytes"] = kv_logical
        sd = torch.tensor(pairs, dtype=torch.int32, device=dev)
        kp, vp = pools[0]

        def cow():
            PK.pkv_copy_blocks(kp, vp, sd)
        cow()
        torch.cuda.synchronize()
        cow_us = _timed(cow, reps, stream)
        cow_bytes = 2 * 2 * len(pairs) * Hkv * P * D * 2
        res.update({"cow_pairs": len(pairs), "cow_us": round(cow_us, 2),
                    "cow_gbps_read_plus_write": round(cow_bytes / cow_us / 1e3, 1)})
        # the same decode with the fork groups named: each group's shared prompt
        # blocks are read once for its 8 samples (pkv_attention_decode_shared)
        gsd = torch.from_numpy(w.group_start).to(dev)
        sws = torch.empty(max(PK.pkv_attention_decode_shared_workspace_bytes(len(seqs), Hq, D, mcl), 256),
                          dtype=torch.uint8, device=dev)
        splan = torch.empty(max(PK.pkv_decode_shared_plan_bytes(len(seqs), mcl), 256), dtype=torch.uint8,
                            device=dev)

        def shared_all():
            # one shared-prefix plan per step, used by every layer
            PK.pkv_decode_shared_plan(splan, td, ld, gsd, Hq, Hkv, mcl, PK.PKV_BF16)
            for kp, vp in pools:
                PK.pkv_attention_decode_shared_planned(out, q, kp, vp, td, ld, mcl, scale, splan, workspace=sws)

        def shared_self_planned():
            for kp, vp in pools:
                PK.pkv_attention_decode_shared(out, q, kp, vp, td, ld, gsd, mcl, scale, workspace=sws)
        shared_all()
        shared_self_planned()
        torch.cuda.synchronize()
        sh_us = _timed(shared_all, reps, stream) / L
        sh_self_us = _timed(shared_self_planned, reps, stream) / L
        res.update({"shared_decode_us_per_layer": round(sh_us, 2),
                    "shared_decode_unique_gbps": round(res["kv_unique_bytes"] / sh_us / 1e3, 1),
                    "shared_decode_hbm_peak_frac": round(res["kv_unique_bytes"] / sh_us / 1e3 / HBM_PEAK_GBPS, 4),
                    "shared_over_plain_speedup": round(dec_us / sh_us, 3),
                    "shared_self_planned_us_per_layer": round(sh_self_us, 2),
                    "shared_kernels": "shared_plans_kernel once per step (shared prefixes, then the tails' plan) "
                                      "+ per layer decode_shared_mfma_kernel (shared prompt blocks on the matrix "
                                      "cores) and decode_valu_kernel (each sample's tail, merge of split rows "
                                      "inside)"})
        # the same batch over float32 pools (2 layers of the same tables): plain
        # decode, and shared-prefix decode (the shared blocks on the fp32 matrix
        # cores, then the samples' tails on the vector-ALU kernel)
        fpools = [(torch.randn(NB, Hkv, P, D, generator=gen, device=dev),
                   torch.randn(NB, Hkv, P, D, generator=gen, device=dev)) for _ in range(2)]
        q32 = torch.randn(len(seqs), Hq, D, generator=gen, device=dev)
        out32 = torch.empty_like(out)
        plan32 = PK.plan_for(ld, Hq, Hkv, MB, mcl, PK.PKV_F32)
        splan32 = torch.empty_like(splan)

        def plain_f32_all():
            for kp, vp in fpools:
                PK.pkv_attention_decode(out32, q32, kp, vp, td, ld, mcl, scale, workspace=ws, plan=plan32)

        def shared_f32_all():
            PK.pkv_decode_shared_plan(splan32, td, ld, gsd, Hq, Hkv, mcl, PK.PKV_F32)
            for kp, vp in fpools:
                PK.pkv_attention_decode_shared_planned(out32, q32, kp, vp, td, ld, mcl, scale, splan32,
                                                       workspace=sws)
        plain_f32_all()
        shared_f32_all()
        torch.cuda.synchronize()
        p32_us = _timed(plain_f32_all, reps, stream) / len(fpools)
        s32_us = _timed(shared_f32_all, reps, stream) / len(fpools)
        u32 = res["kv_unique_bytes"] * 2
        res.update({"decode_f32_us_per_layer": round(p32_us, 2),
                    "shared_decode_f32_us_per_layer": round(s32_us, 2),
                    "shared_decode_f32_unique_gbps": round(u32 / s32_us / 1e3, 1),
                    "shared_decode_f32_hbm_peak_frac": round(u32 / s32_us / 1e3 / HBM_PEAK_GBPS, 4),
                    "shared_f32_over_plain_speedup": round(p32_us / s32_us, 3),
                    "shared_f32_kernels": "shared_plans_kernel once per step + decode_shared_f32_kernel and "
                                          "decode_valu_kernel<float> per layer"})
    if name == "long":
        cs = w.chunk_seqs
        clens = np.array([alloc.seq_block_table(s)[1] for s in cs], dtype=np.int32)
        cmb = int(-(-clens.max() // P))
        ct, _ = alloc.block_tables(cs, cmb)
        qsl = torch.from_numpy(w.chunk_query_start_loc).to(dev)
        nq = np.diff(w.chunk_query_start_loc)
        cq = randn(int(nq.sum()), Hq, D)
        cout = torch.empty(int(nq.sum()), Hq, D, dtype=torch.float32, device=dev)
        ctd, cld = torch.from_numpy(ct).to(dev), torch.from_numpy(clens).to(dev)

        def prefill_all():
            for kp, vp in pools:
                PK.pkv_attention_prefill_chunk(cout, cq, qsl, int(nq.max()), kp, vp, ctd, cld, int(clens.max()),
                                               scale)
        prefill_all()
        torch.cuda.synchronize()
        pf_us = _timed(prefill_all, reps, stream) / L
        # causal flops: q.k and p.v, 2 flops per multiply-add, per (query, head, visible key, dim)
        keys = sum(int(c) * int(n) - int(n) * (int(n) - 1) // 2 for c, n in zip(clens, nq))
        flops = 4 * Hq * D * keys
        # the bf16 kernel issues the P.V products twice (the probability as a
        # bf16 pair, for the 2e-3 bar): 1.5x the credited matrix work
        res.update({"prefill_us_per_layer": round(pf_us, 2), "prefill_tflops": round(flops / pf_us / 1e6, 1),
                    "prefill_mfma_peak_frac": round(flops / pf_us / 1e6 / 2500.0, 4),
                    "prefill_issued_mfma_tflops": round(1.5 * flops / pf_us / 1e6, 1),
                    "prefill_tokens_per_s_per_layer": round(int(nq.sum()) / pf_us * 1e6, 1),
                    "prefill_kernel": "prefill_chunk_mfma_kernel"})
        # the step's mix as one pass: each layer's prefill on a second stream,
        # launched before that layer's decode on this one (the decode units
        # take the CUs that the prefill workgroups leave as they finish)
        side = torch.cuda.Stream()

        def mixed_all():
            start = torch.cuda.Event()
            start.record(stream)
            side.wait_event(start)
            for kp, vp in pools:
                PK.pkv_attention_prefill_chunk(cout, cq, qsl, int(nq.max()), kp, vp, ctd, cld, int(clens.max()),
                                               scale, stream=side)
                PK.pkv_attention_decode(out, q, kp, vp, td, ld, mcl, scale, workspace=ws, plan=plan, stream=stream)
            done = torch.cuda.Event()
            done.record(side)
            stream.wait_event(done)
        mixed_all()
        torch.cuda.synchronize()
        mix_us = _timed(mixed_all, reps, stream) / L
        res.update({"mixed_step_us_per_layer": round(mix_us, 2),
                    "mixed_step_over_sequential": round((dec_us + pf_us) / mix_us, 3)})
        # the same chunks over float32 pools (2 layers of the same tables): the
        # fp32 matrix-core kernel, against the fp32 MFMA peak
        fpools = [(torch.randn(NB, Hkv, P, D, generator=gen, device=dev),
                   torch.randn(NB, Hkv, P, D, generator=gen, device=dev)) for _ in range(2)]
        cq32 = torch.randn(int(nq.sum()), Hq, D, generator=gen, device=dev)
        cout32 = torch.empty_like(cout)

        def prefill_f32_all():
            for kp, vp in fpools:
                PK.pkv_attention_prefill_chunk(cout32, cq32, qsl, int(nq.max()), kp, vp, ctd, cld, int(clens.max()),
                                               scale)
        prefill_f32_all()
        torch.cuda.synchronize()
        pf32_us = _timed(prefill_f32_all, reps, stream) / len(fpools)
        res.update({"prefill_f32_us_per_layer": round(pf32_us, 2),
                    "prefill_f32_tflops": round(flops / pf32_us / 1e6, 1),
                    "prefill_f32_mfma_peak_frac": round(flops / pf32_us / 1e6 / FP32_MFMA_PEAK_TFLOPS, 4),
                    "prefill_f32_kernel": "prefill_chunk_f32_kernel"})
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = secondary_oracle_check(args, w, pools[-1], q, td, ld, tables_h, lens_h, scale,
                                                     locals())
    print(json.dumps(res), flush=True)


def secondary_oracle_check(args, w, pool, q, td, ld, tables_h, lens_h, scale, env):
    """Outside the timed region: the last layer's outputs of a secondary
    workload recomputed on a few rows (its own device inputs, copied to the
    host) by the oracle, reported as max abs error; the oracle's rate beside."""
    import torch
    import paged_kv_cache_171_amd as PK
    from oracle import pkv_oracle as O
    P = 16
    kp, vp = pool
    S, Hq, D = q.shape
    mcl = int(lens_h.max())
    kh, vh, qh = _host_bits(kp), _host_bits(vp), _host_bits(q)
    tl = [list(tables_h[i, :-(-int(c) // P)]) for i, c in enumerate(lens_h)]
    order = np.argsort(-lens_h, kind="stable")
    rows = sorted(set([int(order[0]), int(order[-1])] + [int(x) for x in
                      np.random.default_rng(args.seed).choice(S, size=min(S, 14), replace=False)]))
    cases = []

    def decode_case(outt):
        def fn():
            ref = O.decode_attention(qh[rows], kh, vh, [tl[i] for i in rows], [int(lens_h[i]) for i in rows], scale)
            return ref, outt.cpu().numpy()[rows], len(rows) * Hq
        return fn
    plain = torch.empty(S, Hq, D, dtype=torch.float32, device=q.device)
    PK.pkv_attention_decode(plain, q, kp, vp, td, ld, mcl, scale)
    cases.append(("decode", decode_case(plain)))
    if w.name.startswith("gqa"):
        kp32, vp32 = env["fpools"][-1]
        kh32, vh32, qh32 = _host_bits(kp32), _host_bits(vp32), _host_bits(env["q32"])
        plain32 = torch.empty_like(plain)
        PK.pkv_attention_decode(plain32, env["q32"], kp32, vp32, td, ld, mcl, scale)

        def decode_f32_fn():
            ref = O.decode_attention(qh32[rows], kh32, vh32, [tl[i] for i in rows], [int(lens_h[i]) for i in rows],
                                     scale)
            return ref, plain32.cpu().numpy()[rows], len(rows) * Hq
        cases.append(("decode_f32", decode_f32_fn))
    if w.name == "fork":
        shared = torch.empty_like(plain)
        PK.pkv_attention_decode_shared_planned(shared, q, kp, vp, td, ld, mcl, scale, env["splan"],
                                               workspace=env["sws"])
        cases.append(("shared_decode", decode_case(shared)))
        kp32, vp32 = env["fpools"][-1]
        kh32, vh32, qh32 = _host_bits(kp32), _host_bits(vp32), _host_bits(env["q32"])
        shared32 = torch.empty_like(plain)
        PK.pkv_attention_decode_shared_planned(shared32, env["q32"], kp32, vp32, td, ld, mcl, scale, env["splan32"],
                                               workspace=env["sws"])

        def shared_f32_fn():
            ref = O.decode_attention(qh32[rows], kh32, vh32, [tl[i] for i in rows], [int(lens_h[i]) for i in rows],
                                     scale)
            return ref, shared32.cpu().numpy()[rows], len(rows) * Hq
        cases.append(("shared_decode_f32", shared_f32_fn))
    if w.name == "long":
        cout, cq, ct, clens, qsl = env["cout"], env["cq"], env["ct"], env["clens"], w.chunk_query_start_loc
        cqh = _host_bits(cq)
        ctl = [list(ct[i, :-(-int(c) // P)]) for i, c in enumerate(clens)]

        def prefill_fn():
            # the first chunk, all of its queries
            a, b = int(qsl[0]), int(qsl[1])
            ref = O.prefill_chunk_attention(cqh[a:b], np.array([0, b - a], dtype=np.int32), kh, vh, ctl[:1],
                                            [int(clens[0])], scale)
            return ref, cout.cpu().numpy()[a:b], (b - a) * Hq
        kp32, vp32 = env["fpools"][-1]
        kh32, vh32, cqh32, cout32 = _host_bits(kp32), _host_bits(vp32), _host_bits(env["cq32"]), env["cout32"]

        def prefill_f32_fn():
            # the float32 chunk 0's last 64 queries (the longest contexts)
            b = int(qsl[1])
            a = b - 64
            ref = O.prefill_chunk_attention(cqh32[a:b], np.array([0, 64], dtype=np.int32), kh32, vh32, ctl[:1],
                                            [int(clens[0])], scale)
            return ref, cout32.cpu().numpy()[a:b], 64 * Hq
        cases.append(("prefill_f32", prefill_f32_fn))
        cases.append(("prefill", prefill_fn))
    torch.cuda.synchronize()
    return secondary_cpu_check(w.name, cases, args.cpu_seconds)


PCIE5_X16_GBPS = 64.0     # host link peak per direction (PCIe 5.0 x16)


def swap_bench(args):
    """Swap copies of whole 13B-shaped blocks (40 heads x 16 x 128 bf16, K and V:
    320 KiB per block) between a device pool of 8192 blocks and a pinned host
    pool of 2048 blocks: 1024 random blocks out, then 1024 back in.  Beside it,
    one contiguous copy of the same byte count each way by the runtime (the
    host link's practical ceiling)."""
    import torch
    import paged_kv_cache_171_amd as PK
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    H, D, P, NBD, NBH, n = 40, 128, 16, 8192, 2048, 1024
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    kd = torch.randn(NBD, H, P, D, generator=gen, device=dev).to(torch.bfloat16)
    vd = torch.randn(NBD, H, P, D, generator=gen, device=dev).to(torch.bfloat16)
    kh = torch.empty(NBH, H, P, D, dtype=torch.bfloat16).pin_memory()
    vh = torch.empty(NBH, H, P, D, dtype=torch.bfloat16).pin_memory()
    rng = np.random.default_rng(args.seed)
    out_pairs = np.stack([rng.permutation(NBD)[:n], rng.permutation(NBH)[:n]], 1).astype(np.int32)
    in_pairs = np.stack([rng.permutation(NBH)[:n], rng.permutation(NBD)[:n]], 1).astype(np.int32)
    po, pi = torch.from_numpy(out_pairs).to(dev), torch.from_numpy(in_pairs).to(dev)
    reps = max(args.steps, 3)

    def out():
        PK.pkv_swap_blocks(kh, vh, kd, vd, po)

    def back():
        PK.pkv_swap_blocks(kd, vd, kh, vh, pi)
    for _ in range(max(args.warmup, 1)):
        out()
        back()
    torch.cuda.synchronize()
    out_us = _timed(out, reps, stream)
    in_us = _timed(back, reps, stream)
    nbytes = 2 * n * H * P * D * 2
    flat_h = kh.view(-1)[: nbytes // 2]
    flat_d = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev)
    d2h_us = _timed(lambda: flat_h.copy_(flat_d, non_blocking=True), reps, stream)
    h2d_us = _timed(lambda: flat_d.copy_(flat_h, non_blocking=True), reps, stream)
    gb = lambda us: round(nbytes / us / 1e3, 2)
    print(json.dumps({
        "workload": "swap", "kernel": "copy_blocks_kernel (pkv_swap_blocks)", "pairs": n,
        "block_bytes_k_plus_v": 2 * H * P * D * 2, "bytes_per_launch": nbytes,
        "swap_out_us": round(out_us, 1), "swap_out_gbps": gb(out_us),
        "swap_in_us": round(in_us, 1), "swap_in_gbps": gb(in_us),
        "runtime_contiguous_d2h_gbps": gb(d2h_us), "runtime_contiguous_h2d_gbps": gb(h2d_us),
        "roofline": {"bound": "host link", "peak": PCIE5_X16_GBPS, "unit": "GB/s",
                     "swap_out_frac": round(nbytes / out_us / 1e3 / PCIE5_X16_GBPS, 4),
                     "swap_in_frac": round(nbytes / in_us / 1e3 / PCIE5_X16_GBPS, 4)}}), flush=True)


def serve_bench(args):
    """The continuous-batching loop, end to end on one GPU: 256 requests, prompt
    lengths lognormal (median 200, sigma 1) clipped to [1, 1024], output
    lengths lognormal (median 128, sigma 0.8) clipped to [1, 512]; 40 MHA heads
    x 128, bf16, 4 layer pools; at most 64 running requests and 4096 tokens a
    step; a device pool of 1600 blocks (64 requests at their mean final length
    need ~1850), so requests are swapped out to a 512-block pinned host pool
    and back.  Per step: the native step executor (pkv_batch_schedule: the
    scheduler step, the step's indices to the GPU, the decode plan), then per
    layer pkv_batch_layer: the swap copies, the cache writes, causal prefill of
    admitted prompts and decode of the running requests.  Rows and queries are random and reused.  Run once
    under the continuous policy and once under the static one."""
    import torch
    import paged_kv_cache_171_amd as PK
    import pkv_workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L, H, D, P = 4, 40, 128, 16
    w = W.serving(seed=args.seed, num_requests=256, hq=H, hkv=H, d=D, prompt_median=200, output_median=128,
                  sigma=1.0, max_prompt=1024, max_output=512, num_blocks=1600, max_num_seqs=64,
                  max_num_batched_tokens=4096, num_host_blocks=512, with_rows=False)
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    pools = [(randn(w.num_blocks, H, P, D), randn(w.num_blocks, H, P, D)) for _ in range(L)]
    hosts = [(torch.empty(w.num_host_blocks, H, P, D, dtype=torch.bfloat16).pin_memory(),
              torch.empty(w.num_host_blocks, H, P, D, dtype=torch.bfloat16).pin_memory()) for _ in range(L)]
    T = w.max_num_batched_tokens
    qr, kr, vr = randn(T, H, D), randn(T, H, D), randn(T, H, D)
    out = torch.empty(T, H, D, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(D)
    from paged_kv_cache_171_amd import binding as B
    lib, sp = B.LIB, torch.cuda.current_stream().cuda_stream
    mb = int(-(-int((w.prompts + w.outputs).max()) // P))
    ptrs = [(kp.data_ptr(), vp.data_ptr(), kh.data_ptr(), vh.data_ptr()) for (kp, vp), (kh, vh) in zip(pools, hosts)]
    qkvo = (qr.data_ptr(), kr.data_ptr(), vr.data_ptr(), out.data_ptr())
    results = {}
    for name, policy in (("continuous", PK.PKV_SCHED_CONTINUOUS), ("static", PK.PKV_SCHED_STATIC)):
        alloc = PK.BlockAllocator(w.num_blocks, P, w.initial_free_order)
        sched = PK.Scheduler(alloc, w.max_num_seqs, T, policy, w.num_host_blocks)
        for p, o in zip(w.prompts, w.outputs):
            sched.add_request(int(p), int(o))
        batch = PK.Batch(sched, mb, w.num_blocks, w.num_host_blocks, H, H, D)
        info = B._StepInfo()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        steps = tokens = swapped = 0
        while True:
            # one native call schedules the step and moves its indices to the GPU,
            # then one per layer enqueues swaps, cache write, prefill and decode
            B._check(lib.pkv_batch_schedule(batch._h, sp, ctypes.byref(info)))
            n = info.num_prefill + info.num_decode
            if n == 0:
                break
            for kp, vp, kh, vh in ptrs:
                B._check(lib.pkv_batch_layer(batch._h, kp, vp, kh, vh, qkvo[0], qkvo[1], qkvo[2], qkvo[3], scale, sp))
            steps += 1
            tokens += n
            swapped += info.num_swapped_out
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        st = sched.stats()
        results[name] = {"steps": steps, "generated_tokens": tokens, "seconds": round(el, 3),
                         "tokens_per_s": round(tokens / el, 1), "ms_per_step": round(el / steps * 1e3, 3),
                         "slot_utilisation": round(st[1] / (steps * w.max_num_seqs), 4),
                         "swapped_out_requests": swapped}
        del batch
    print(json.dumps({"workload": "serve", "layers": L, "requests": len(w.prompts), "heads": H, "head_dim": D,
                      "max_num_seqs": w.max_num_seqs, "max_num_batched_tokens": T,
                      "device_blocks": w.num_blocks, "host_blocks": w.num_host_blocks,
                      "mean_prompt": round(float(w.prompts.mean()), 1), "mean_output": round(float(w.outputs.mean()), 1),
                      **results,
                      "continuous_over_static": round(results["continuous"]["tokens_per_s"] /
                                                      results["static"]["tokens_per_s"], 3)}), flush=True)


def blocksize_bench(args):
    """Block sizes 8, 16 and 32 on two batches: the 13B-shaped decode (64 seqs,
    40 MHA heads x 128, bf16, lognormal contexts; the vector-ALU kernel, 8
    layer pools) and the grouped-query batch (256 seqs, 64 query / 8 KV heads,
    contexts U[128, 4096]; the matrix-core kernel, which walks 16-key tiles --
    two 8-token blocks or half a 32-token block each; 4 layer pools).  Per
    block size the block-table entries, the slots reserved but unused in each
    sequence's last block (the tail waste of [CB] "PagedAttention: Memoria
    virtual para la KV cache"), and the decode kernel's time and K/V bandwidth
    (each pool 1.2x the blocks needed at that size, shuffled)."""
    import torch
    import paged_kv_cache_171_amd as PK
    import pkv_workloads as W
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    reps = max(args.steps, 3)

    def sweep(make, L, kernel):
        rows = []
        for bs in (8, 16, 32):
            w = make(bs)
            H, Hkv, D = w.num_heads, w.num_kv_heads, w.head_dim
            alloc = PK.BlockAllocator(w.num_blocks, bs, w.initial_free_order)
            for op in w.ops:
                if op[0] == "create":
                    alloc.seq_create()
                elif op[0] == "append":
                    alloc.seq_append_slots(op[1], op[2])
            seqs = w.decode_seqs
            lens = np.array([alloc.seq_block_table(s)[1] for s in seqs], dtype=np.int32)
            MB = int(-(-lens.max() // bs))
            tables, _ = alloc.block_tables(seqs, MB)
            pools = [(torch.randn(w.num_blocks, Hkv, bs, D, generator=gen, device=dev).to(torch.bfloat16),
                      torch.randn(w.num_blocks, Hkv, bs, D, generator=gen, device=dev).to(torch.bfloat16))
                     for _ in range(L)]
            q = torch.randn(len(seqs), H, D, generator=gen, device=dev).to(torch.bfloat16)
            out = torch.empty(len(seqs), H, D, dtype=torch.float32, device=dev)
            td, ld = torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev)
            mcl = int(lens.max())
            ws = PK.workspace_for(len(seqs), H, D, mcl, device=dev)
            plan = PK.plan_for(ld, H, Hkv, MB, mcl, PK.PKV_BF16, block_size=bs)

            def decode_all():
                for kp, vp in pools:
                    PK.pkv_attention_decode(out, q, kp, vp, td, ld, mcl, 1.0 / math.sqrt(D), workspace=ws,
                                            plan=plan)
            decode_all()
            torch.cuda.synchronize()
            dec_us = _timed(decode_all, reps, stream) / L
            blocks = int(sum(-(-int(c) // bs) for c in lens))
            kv = int(lens.sum()) * 2 * Hkv * D * 2
            rows.append({"block_size": bs, "pool_blocks": w.num_blocks, "table_entries": blocks,
                         "table_bytes_padded": len(seqs) * MB * 4,
                         "tail_waste_frac": round(1 - int(lens.sum()) / (blocks * bs), 4),
                         "decode_us_per_layer": round(dec_us, 2), "decode_kv_gbps": round(kv / dec_us / 1e3, 1),
                         "decode_hbm_peak_frac": round(kv / dec_us / 1e3 / HBM_PEAK_GBPS, 4)})
            del pools
            torch.cuda.empty_cache()
        return {"kernel": kernel, "layers": L, "sweep": rows}

    res = {"workload": "blocksize",
           "13b": dict(num_seqs=64, heads="40/40", head_dim=128,
                       **sweep(lambda bs: W.shaped_13b(seed=args.seed, with_rows=False, block_size=bs), 8,
                               "decode_valu_kernel<bf16,128,BS> (merge inside)")),
           "gqa": dict(num_seqs=256, heads="64/8", head_dim=128,
                       **sweep(lambda bs: W.gqa(with_rows=False, block_size=bs), 4,
                               "decode_group_mfma_kernel<128,BS> (merge inside)"))}
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the library has no multi-GPU path (one process, one device)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    if args.workload == "swap":
        swap_bench(args)
        return
    if args.workload == "serve":
        serve_bench(args)
        return
    if args.workload == "blocksize":
        blocksize_bench(args)
        return
    if args.workload == "probes":
        probes_bench(args)
        return
    if args.workload != "13b":
        secondary(args)
        return

    import torch
    import paged_kv_cache_171_amd as PK
    from paged_kv_cache_171_amd import binding as B
    import pkv_workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L, S, H, D, P = args.layers, 64, 40, 128, 16

    lens0 = W.shaped_13b_lengths(seed=args.seed, num_seqs=S)
    total_steps = args.warmup + args.steps
    need = sum(-(-int(c) // P) for c in lens0)
    NB = int(math.ceil(1.2 * need))
    perm = np.random.default_rng(args.seed + 1000).permutation(NB).astype(np.int32)
    MB = -(-(int(lens0.max()) + total_steps) // P)

    # host allocator with the prompt tokens of every sequence already cached
    alloc = PK.BlockAllocator(NB, P, perm)
    seqs = [alloc.seq_create() for _ in range(S)]
    for s, c in zip(seqs, lens0):
        alloc.seq_append_slots(s, int(c) - 1)

    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)

    k_pools = [randn(NB, H, P, D) for _ in range(L)]
    v_pools = [randn(NB, H, P, D) for _ in range(L)]
    q = [randn(S, H, D) for _ in range(L)]
    k_new = [randn(S, H, D) for _ in range(L)]
    v_new = [randn(S, H, D) for _ in range(L)]
    out = [torch.empty(S, H, D, dtype=torch.float32, device=dev) for _ in range(L)]
    max_ctx_cap = int(lens0.max()) + total_steps
    ws_bytes = PK.pkv_attention_workspace_bytes(S, H, D, max_ctx_cap)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    plan_bytes = PK.pkv_decode_plan_bytes(S, max_ctx_cap)

    # The step's indices (slots, tables, lengths, copy pairs) travel in one
    # packed buffer: pinned staging on the host, one set per step of a phase
    # (the host runs steps ahead of the GPU, so a set must not be refilled
    # while an earlier step's copy may still read it; the warm-up and the timed
    # phase are separated by a synchronize, so the timed steps reuse the
    # warm-up's sets), one copy per step into the device set on the launch
    # stream.  (A side stream that copies and plans step k while step k-1's
    # layers run made the step 10-20 % slower on this GPU.)
    def a256(n):
        return (n + 255) // 256 * 256
    off_tables = a256(S * 8)
    off_lens = off_tables + a256(S * MB * 4)
    off_pairs = off_lens + a256(S * 4)
    packed = off_pairs + a256(S * 8)

    def views(buf):
        return (buf[off_tables:off_tables + S * MB * 4].view(torch.int32).view(S, MB),
                buf[off_lens:off_lens + S * 4].view(torch.int32), buf[:S * 8].view(torch.int64),
                buf[off_pairs:off_pairs + S * 8].view(torch.int32).view(S, 2))
    staging = [torch.zeros(packed, dtype=torch.uint8).pin_memory() for _ in range(max(args.warmup, args.steps))]
    buf_d = torch.zeros(packed, dtype=torch.uint8, device=dev)
    plan = torch.zeros(max(plan_bytes, 256), dtype=torch.uint8, device=dev)
    tables_d, lens_d, slots_d, pairs_d = views(buf_d)
    scale = 1.0 / math.sqrt(D)
    torch.cuda.synchronize()

    lib = B.LIB
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    ones = np.ones(S, dtype=np.int32)
    kp = [(k_pools[l].data_ptr(), v_pools[l].data_ptr()) for l in range(L)]
    kvn = [(k_new[l].data_ptr(), v_new[l].data_ptr()) for l in range(L)]
    qp = [q[l].data_ptr() for l in range(L)]
    op = [out[l].data_ptr() for l in range(L)]
    BF16 = PK.PKV_BF16

    host_us = []

    def step(k, events=None):
        """Step k of its phase; events: a (start, end) pair recorded around the
        step's L decode launches."""
        # (a1) host: reserve one slot per sequence, refresh the tables
        h0 = time.perf_counter()
        slots, pairs = alloc.seq_append_slots_batch(seqs, ones)
        t, ln = alloc.block_tables(seqs, MB)
        tables_h, lens_h, slots_h, pairs_h = views(staging[k])
        slots_h.numpy()[:] = slots
        tables_h.numpy()[:] = t
        lens_h.numpy()[:] = ln
        n_pairs = len(pairs)
        if n_pairs:
            pairs_h.numpy()[:n_pairs] = pairs
        max_ctx = int(ln.max())
        if events is not None:
            host_us.append((time.perf_counter() - h0) * 1e6)
        buf_d.copy_(staging[k], non_blocking=True)
        # the decode plan depends only on this step's lengths: built once, used by every layer
        B._check(lib.pkv_decode_plan(plan.data_ptr(), plan.numel(), lens_d.data_ptr(), S, H, H, MB, P, max_ctx, BF16,
                                     sp))
        for l in range(L):
            if n_pairs:   # (a2) copy-on-write (none arise in this workload)
                B._check(lib.pkv_copy_blocks(kp[l][0], kp[l][1], pairs_d.data_ptr(), n_pairs, NB, H, D, P, BF16, sp))
            # (a3, a4, a5) this step's K/V written at their slots inside the paged
            # decode attention launch, then the partition merge
            if events is not None and l == 0:
                events[0].record(stream)
            B._check(lib.pkv_attention_decode_append(op[l], qp[l], kvn[l][0], kvn[l][1], slots_d.data_ptr(),
                                                     kp[l][0], kp[l][1], tables_d.data_ptr(), MB, lens_d.data_ptr(),
                                                     S, H, H, D, P, NB, max_ctx, scale, BF16, plan.data_ptr(),
                                                     plan.numel(), ws.data_ptr(), ws.numel(), sp))
            if events is not None and l == L - 1:
                events[1].record(stream)
        return ln

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    # the L decode launches of each step are bracketed by one pair of events
    # (events around every launch add two markers per layer to the step and
    # read a few microseconds high each)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    step_lens = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step_lens.append(step(k, ev[k]))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # every output row of the last step is finite: each sequence's slot matched
    # its last token and every table entry was in the pool
    for l in range(L):
        if not bool(torch.isfinite(out[l]).all()):
            raise SystemExit(f"bench: non-finite attention output in layer {l}")

    # algorithmic bytes of one decode launch: K and V of every live token once
    # (the new token's from the step's rows), the new K/V rows written to the
    # pool, plus q, the fp32 output, the table entries in use, the lengths and
    # the slots
    kv_bytes = [int(ln.sum()) * 2 * H * D * 2 for ln in step_lens]
    other = [S * 2 * H * D * 2 + S * H * D * 2 + S * H * D * 4 + int(sum(-(-int(c) // P) for c in ln)) * 4 + S * 4 +
             S * 8 for ln in step_lens]
    dec_ms = [ev[k][0].elapsed_time(ev[k][1]) for k in range(args.steps)]
    launches = args.steps * L
    alg_bytes_total = sum((kv + o) * L for kv, o in zip(kv_bytes, other))
    dec_s_total = sum(dec_ms) / 1e3
    achieved = alg_bytes_total / dec_s_total / 1e9
    avg_launch_us = dec_s_total / launches * 1e6
    step_s = ms_per_step / 1e3
    kv_gbps = (sum(kv_bytes) / args.steps) * L / step_s / 1e9

    traffic = stored_traffic(alg_bytes_total / launches)
    res = {
        "metric": METRIC,
        "value": round(S / step_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "13b-shaped decode step: 64 seqs, 40 MHA heads x head_dim 128, bf16 K/V/q, "
                        "lognormal ctx (median 200, sigma 1) clipped [1,2048], block 16, pool 1.2x shuffled, "
                        f"{L} layer pools",
            "global_batch": S, "layers": L, "mean_ctx": round(float(np.mean([ln.mean() for ln in step_lens])), 1),
            "partition_tokens": 1024, "parallelism": "none (1 GPU)"},
        "kv_gbps_step": round(kv_gbps, 1),
        "hbm_peak_frac_step": round(kv_gbps / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": "decode_valu_kernel<bf16,128,16> (with the cache write and the merge of split contexts)",
                     "avg_launch_us": round(avg_launch_us, 2),
                     "alg_bytes_per_launch": round(alg_bytes_total / launches)},
        # (a1) on the host, while the GPU runs earlier steps: slot reservation
        # for the 64 sequences and the table refresh in the native allocator
        # (one binding call each), and the staging fill
        "host_slots_tables_us_per_step": round(float(np.median(host_us)), 1),
    }
    if not args.no_cpu_baseline:
        # the oracle on the last timed step's inputs, compared with its outputs
        tables_last, _ = alloc.block_tables(seqs, MB)
        lens_last = step_lens[-1]
        tl = [list(tables_last[i, :-(-int(c) // P)]) for i, c in enumerate(lens_last)]

        def layer_tensors(l):
            return L if l is None else (q[l], k_pools[l], v_pools[l], out[l])
        res["cpu_baseline"] = cpu_baseline(layer_tensors, tl, lens_last, np.float32(scale), args.cpu_seconds, 2e-3)
    # a second denominator: the best streaming read measured on this GPU
    del k_pools, v_pools
    torch.cuda.empty_cache()
    probe = read_probes(stream)
    res["roofline"]["read_probe_gbps"] = round(probe["best_gbps"], 1)
    res["roofline"]["read_probe"] = probe
    res["roofline"]["frac_of_read_probe"] = round(achieved / probe["best_gbps"], 4)
    print(json.dumps(res), flush=True)


def _median_us(fn, stream, reps):
    import torch
    fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    return float(np.median(ts))


STREAM_MODES = {0: "nt x4", 1: "nt x8", 2: "nt x16", 3: "plain x4", 4: "plain x8", 5: "plain x16"}


def read_probes(stream, reps: int = 10, gib: int = 4, sweep: bool = False) -> dict:
    """GB/s of streaming reads of one 4 GiB buffer on this GPU (median of `reps`
    runs each, HIP events on `stream`): the hand-written stream_read_kernel
    (libpkv_probes.so) over launch shapes (16-byte loads, 4/8/16 in flight per
    thread, non-temporal or ordinary, 1024..8192 workgroups of 256 threads),
    and torch.mv, the BLAS gemv, over the same bytes as a 65536 x 32768 bf16
    matrix.  The best of all is the measured read ceiling."""
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_171_amd", "libpkv_probes.so"))
    lib.pkvprobe_stream_read.restype = ctypes.c_int
    lib.pkvprobe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_void_p]
    nbytes = gib << 30
    m = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    grids = (1024, 2048, 4096, 8192) if sweep else (2048, 4096)
    modes = tuple(STREAM_MODES) if sweep else (1, 4)
    sink = torch.zeros(max(grids) * 256, dtype=torch.int32, device="cuda")
    sp = stream.cuda_stream
    res = {"bytes": nbytes, "stream_read": {}}
    best = (0.0, None)
    for mode in modes:
        for grid in grids:
            def run(mode=mode, grid=grid):
                rc = lib.pkvprobe_stream_read(m.data_ptr(), nbytes, grid, mode, sink.data_ptr(), sp)
                if rc != 0:
                    raise RuntimeError(f"stream_read launch failed: {rc}")
            gbps = nbytes / _median_us(run, stream, reps) / 1e3
            res["stream_read"][f"{STREAM_MODES[mode]} grid {grid}"] = round(gbps, 1)
            if gbps > best[0]:
                best = (gbps, f"stream_read_kernel {STREAM_MODES[mode]}, grid {grid}")
    mat = m.view(65536, nbytes // 2 // 65536)
    v = torch.ones(mat.shape[1], dtype=torch.bfloat16, device="cuda")
    mv = nbytes / _median_us(lambda: torch.mv(mat, v), stream, reps) / 1e3
    res["torch_mv_gbps"] = round(mv, 1)
    if mv > best[0]:
        best = (mv, "torch.mv")
    res["best_gbps"] = best[0]
    res["best"] = best[1]
    del m, mat, v, sink
    torch.cuda.empty_cache()
    return res


def mfma_probe(stream, reps: int = 10) -> dict:
    """TFLOP/s of the bf16 matrix cores with no memory traffic (mfma_rate_kernel:
    chains of v_mfma_f32_16x16x32_bf16, 256-thread workgroups, 1024 or 2048 of
    them, i.e. 4 or 8 waves per SIMD), medians of `reps` runs."""
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_171_amd", "libpkv_probes.so"))
    lib.pkvprobe_mfma_rate.restype = ctypes.c_int
    lib.pkvprobe_mfma_rate.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_void_p]
    out = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    res = {}
    for grid in (1024, 2048):
        for chains in (1, 2):
            iters = 4096 // chains

            def run(grid=grid, chains=chains, iters=iters):
                rc = lib.pkvprobe_mfma_rate(out.data_ptr(), grid, iters, chains, stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"mfma_rate launch failed: {rc}")
            flops = grid * 4 * iters * chains * 16384
            res[f"{chains} chain(s), {grid // 256} waves/SIMD"] = round(flops / _median_us(run, stream, reps) / 1e6, 1)
    # the 32 x 32 x 16 instruction (32768 flops each)
    lib.pkvprobe_mfma32_rate.restype = ctypes.c_int
    lib.pkvprobe_mfma32_rate.argtypes = lib.pkvprobe_mfma_rate.argtypes
    for grid in (1024, 2048):
        for chains in (1, 2):
            iters = 2048 // chains

            def run_wide(grid=grid, chains=chains, iters=iters):
                rc = lib.pkvprobe_mfma32_rate(out.data_ptr(), grid, iters, chains, stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"mfma32_rate launch failed: {rc}")
            flops = grid * 4 * iters * chains * 32768
            res[f"32x32x16: {chains} chain(s), {grid // 256} waves/SIMD"] = round(
                flops / _median_us(run_wide, stream, reps) / 1e6, 1)
    res["unit"] = "TFLOP/s"
    res["dense_bf16_peak"] = 2500.0
    # the fp32 matrix cores (v_mfma_f32_16x16x4_f32, 2048 flops each)
    lib.pkvprobe_mfma_f32_rate.restype = ctypes.c_int
    lib.pkvprobe_mfma_f32_rate.argtypes = lib.pkvprobe_mfma_rate.argtypes
    for grid in (1024, 2048):
        for chains in (1, 2):
            iters = 4096 // chains

            def run32(grid=grid, chains=chains, iters=iters):
                rc = lib.pkvprobe_mfma_f32_rate(out.data_ptr(), grid, iters, chains, stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"mfma_f32_rate launch failed: {rc}")
            flops = grid * 4 * iters * chains * 2048
            res[f"fp32: {chains} chain(s), {grid // 256} waves/SIMD"] = round(
                flops / _median_us(run32, stream, reps) / 1e6, 1)
    res["dense_fp32_peak"] = FP32_MFMA_PEAK_TFLOPS
    return res


def overlap_probe(stream, reps: int = 5) -> dict:
    """How far matrix-core work of some waves and vector work (fma + exp2, the
    softmax's kind) of other waves on the same SIMD overlap (overlap_kernel:
    roles by wave slot, so every SIMD holds both): the mixed launch against
    each role's waves alone, at 4 and 8 waves per SIMD.  overlap = (sum of the
    two alone - mixed) / the shorter alone: 1 is full overlap, 0 none."""
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_171_amd", "libpkv_probes.so"))
    lib.pkvprobe_overlap.restype = ctypes.c_int
    lib.pkvprobe_overlap.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_void_p]
    out = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    res = {}
    for grid in (1024, 2048):
        def run(mode, grid=grid):
            rc = lib.pkvprobe_overlap(out.data_ptr(), grid, mode, 2048, 1024, stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"overlap probe launch failed: {rc}")
        t = {m: _median_us(lambda m=m: run(m), stream, reps) for m in range(5)}
        run(2)
        torch.cuda.synchronize()
        share = float((out[:grid * 256].view(-1, 64)[:, 0] > 1e29).float().mean())
        alone = t[3] + t[4]
        res[f"{grid // 256} waves/SIMD"] = {
            "all_matrix_us": round(t[0], 1), "all_vector_us": round(t[1], 1), "mixed_us": round(t[2], 1),
            "matrix_waves_alone_us": round(t[3], 1), "vector_waves_alone_us": round(t[4], 1),
            "vector_share": round(share, 3), "overlap": round((alone - t[2]) / min(t[3], t[4]), 3)}
    return res


def probes_bench(args):
    """The ceilings behind the figures: the streaming-read sweep (read_probes),
    the bf16 matrix-core rate with no memory traffic (mfma_probe), and a
    read-only probe of the 13B-shaped decode's own access
    pattern -- the same 64 lognormal contexts, tables and 40 layer pools of
    whole 4 KiB K and V tiles, one workgroup per (16-block chunk, head), chunks
    longest first, nothing computed -- timed over the 40 layers."""
    import torch
    import paged_kv_cache_171_amd as PK
    import pkv_workloads as W
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    res = {"workload": "probes", "read": read_probes(stream, sweep=True), "mfma": mfma_probe(stream),
           "overlap": overlap_probe(stream)}
    L, H, D, P = args.layers, 40, 128, 16
    w = W.shaped_13b(seed=args.seed, with_rows=False)
    alloc = PK.BlockAllocator(w.num_blocks, P, w.initial_free_order)
    for op in w.ops:
        if op[0] == "create":
            alloc.seq_create()
        elif op[0] == "append":
            alloc.seq_append_slots(op[1], op[2])
    seqs = w.decode_seqs
    lens = np.array([alloc.seq_block_table(s_)[1] for s_ in seqs], dtype=np.int32)
    MB = int(-(-lens.max() // P))
    tables, _ = alloc.block_tables(seqs, MB)
    nblk = -(-lens // P)
    work = [(s_, c) for s_ in range(len(seqs)) for c in range(-(-int(nblk[s_]) // 16))]
    work.sort(key=lambda sc: -min(16, int(nblk[sc[0]]) - 16 * sc[1]))       # full chunks first
    work_d = torch.tensor(work, dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    pools = [(torch.randn(w.num_blocks, H, P, D, generator=gen, device=dev).to(torch.bfloat16),
              torch.randn(w.num_blocks, H, P, D, generator=gen, device=dev).to(torch.bfloat16)) for _ in range(L)]
    td, ld = torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev)
    sink = torch.zeros(len(work) * H * 4, dtype=torch.int32, device=dev)
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_171_amd", "libpkv_probes.so"))
    lib.pkvprobe_tile_read.restype = ctypes.c_int
    sp = stream.cuda_stream

    def all_layers():
        for kp, vp in pools:
            rc = lib.pkvprobe_tile_read(ctypes.c_void_p(kp.data_ptr()), ctypes.c_void_p(vp.data_ptr()),
                                        ctypes.c_void_p(td.data_ptr()), MB, ctypes.c_void_p(ld.data_ptr()), P,
                                        ctypes.c_void_p(work_d.data_ptr()), len(work), H, 4096,
                                        ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(sp))
            if rc != 0:
                raise RuntimeError(f"tile_read launch failed: {rc}")
    us = _median_us(all_layers, stream, max(args.steps, 5)) / L
    kv = int(lens.sum()) * 2 * H * D * 2
    res["tile_read"] = {"kernel": "tile_read_kernel (one workgroup per 16-block chunk and head, 4 waves)",
                        "layers": L, "num_seqs": len(seqs), "cached_tokens": int(lens.sum()),
                        "kv_bytes_per_layer": kv, "us_per_layer": round(us, 2),
                        "gbps": round(kv / us / 1e3, 1), "hbm_peak_frac": round(kv / us / 1e3 / HBM_PEAK_GBPS, 4)}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
